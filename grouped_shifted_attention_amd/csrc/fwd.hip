// S2-Attn forward kernel for gfx950.
//
// One workgroup computes BM = 32*NW rows (a "q tile") of one unit (batch b,
// q head h, group g); wave w owns rows 32w..32w+31 of the tile.  The unit's
// local row j lives at original position (g*G + j + shift_h) mod N, so the
// roll by -shift_h and the cut into groups are only address arithmetic
// (AIMech "LongLoRA and Shifted Sparse Attention (S^2-Attn)", opening
// definition); the output row is written back to the same original position,
// which is the roll back by +shift_h.
//
// Per k/v tile of BN = 64 keys, loaded straight into LDS (double-buffered;
// the next tile's loads are in flight during the current tile's math):
//   S^T = K Q^T           MFMA, A = K rows from LDS, B = Q held in VGPRs
//   causal mask           only on tiles that cross the wave's diagonal
//   online softmax        exp2 domain; row max/sum need one lane swap (l^32)
//   O^T += V^T P^T        MFMA, A = V^T read transposed (ds_read_b64_tr_b16)
//                         from the row-major V tile, B = P taken straight
//                         from the S^T accumulators
// Computing S^T (not S) leaves each lane with one query row, so the softmax
// statistics and the rescale of O are per-lane scalars.
#include "device_common.hpp"
#include "kernels.hpp"
#include "staging.hpp"

#include <type_traits>

namespace s2a {

namespace {

constexpr int kBN = 64;
constexpr float kLazy = 8.f;  // log2-domain slack before the softmax reference moves

// VCOPY: V reaches LDS as a transposed copy through VGPRs (plain 16-byte
// reads for O^T += V^T P^T); otherwise V is loaded straight into LDS and read
// with the transposing LDS read.
template <int D, int NW, bool ROPE, bool VCOPY>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(FwdArgs a, RopeTable rope) {
  constexpr int BM = NW * 32;
  using TileStage = LdsStage<D, kBN, NW>;
  using VtStage = TransposeStage<D, kBN, NW * 64>;
  // Eight-wave workgroups (one per CU) keep three tiles in LDS and load two
  // ahead; smaller ones (two per CU) keep two and load one ahead.  The VGPR
  // transposed copy of V is always one tile ahead.
  constexpr int NBUF = (NW >= 8 && !VCOPY) ? 3 : 2;
  constexpr int VELEMS = VCOPY ? D * VtStage::TSTR : kBN * D;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NBUF][kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NBUF][VELEMS];
  VtStage vts;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const SwzLane<D> sw(lane);
  const Shape& s = a.s;

  // Work item: heavy (long causal rows) tiles first within a unit; units
  // contiguous per XCD.
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int unit = logical / a.tiles;
  const int t = a.tiles - 1 - (logical - unit * a.tiles);
  const int g = unit % s.NG;
  const int bh = unit / s.NG;
  const int h = bh % s.H;
  const int b = bh / s.H;
  const int sh = (h >= (s.H >> 1)) ? s.shift : 0;
  const int kvh = h / (s.H / s.Hkv);
  const int base = g * s.G + sh;
  const long long kv_row = (long long)s.Hkv * D;
  const uint16_t* kb_ptr = a.k + (long long)b * s.N * kv_row + (long long)kvh * D;
  const uint16_t* vb_ptr = a.v + (long long)b * s.N * kv_row + (long long)kvh * D;

  // ---- this lane's query row, held as MFMA B operands ----
  const int wave_q0 = t * BM + wave * 32;
  const int qi = wave_q0 + l32;
  const bool qvalid = qi < s.G;
  const int qpos = qvalid ? orig_pos(base, qi, s.N) : 0;
  const long long qoff = ((long long)(b * (long long)s.N + qpos) * s.H + h) * D;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 raw = qvalid ? ld16(a.q + qoff + kk * 16 + hh * 8) : zero_u4();
    if constexpr (ROPE) {
      float x[8];
      unpack8(raw, x);
      rope_rotate8(x, qpos, rope.rev, kk * 16 + hh * 8, false);
      raw = pack8(x);
    }
    qf[kk] = as_bf16x8(raw);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = zero16();
  float m_run = -INFINITY;  // running max of scaled logits (log2 domain)
  float l_run = 0.f;        // this lane's half of the running row sum

  const int rows_end = min((t + 1) * BM, s.G);
  const int ntiles = (rows_end + kBN - 1) / kBN;

  const TileStage ts(wave, lane, (int)kv_row);
  // K and V tiles go straight from global memory into the swizzled LDS
  // tiles; rows past the group end point at the group's last row (their
  // keys are masked, so the values never contribute).
  auto load_tile = [&](int n) {
    const int key0 = n * kBN;
    const int buf = n % NBUF;
    const uint16_t* kt = contig_tile(kb_ptr, kv_row, base, key0, kBN, s.G, s.N);
    auto rows = [&](const uint16_t* head0) {
      return [=, &s](int row) {
        const int j = min(key0 + row, s.G - 1);
        return head0 + orig_pos(base, j, s.N) * kv_row;
      };
    };
    if (kt != nullptr) {
      ts.load_contig(kt, Ks[buf], wave);
      if constexpr (VCOPY)
        vts.load_contig(tid, vb_ptr + (kt - kb_ptr), (int)kv_row);
      else
        ts.load_contig(vb_ptr + (kt - kb_ptr), Vs[buf], wave);
    } else {
      ts.load_rows(rows(kb_ptr), Ks[buf], wave, lane);
      if constexpr (VCOPY)
        vts.load_rows(tid, rows(vb_ptr));
      else
        ts.load_rows(rows(vb_ptr), Vs[buf], wave, lane);
    }
  };

  // One k/v tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  MASK is set
  // only for tiles that reach past this wave's first row (the diagonal).
  auto compute = [&](int n, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int cur = n % NBUF;
    const int key0 = n * kBN;
    // S^T: the two 32-key blocks are independent accumulators, interleaved
    // so back-to-back MFMAs never wait on each other; K fragments are read
    // from LDS one k-step ahead.
    f32x16 sc[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) sc[kb] = zero16();
    {
      const uint16_t* kt = Ks[cur];
      bf16x8 kf[2][kBN / 32];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) kf[0][kb] = sw.row(kt, kb * 32, 0);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + 1 < D / 16) {
#pragma unroll
          for (int kb = 0; kb < kBN / 32; ++kb)
            kf[(kk + 1) & 1][kb] = sw.row(kt, kb * 32, kk + 1);
        }
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb) sc[kb] = mfma32x32x16(kf[kk & 1][kb], qf[kk], sc[kb]);
      }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j > qi) sc[kb][r] = -INFINITY;
        }
    }
    // Online softmax in the exp2 domain with a lazily moved reference: the
    // accumulators are rescaled only when some row's max exceeds the current
    // reference by more than kLazy (so p <= 2^kLazy); otherwise the stale
    // reference stays, which changes nothing in exact arithmetic.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = half_max(mx) * a.scale_log2;
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
    }
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(sc[kb][r] * a.scale_log2 - m_run);
        sc[kb][r] = pv;
        rs += pv;
      }
    l_run += rs;
    // P as bf16 B operands: accumulator elements 0..7 and 8..15 of each
    // 32-key block are the two 16-key halves of the reduction.
    bf16x8 pb[kBN / 32][2];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      pb[kb][0] = cvt8(f32x8{sc[kb][0], sc[kb][1], sc[kb][2], sc[kb][3],
                             sc[kb][4], sc[kb][5], sc[kb][6], sc[kb][7]});
      pb[kb][1] = cvt8(f32x8{sc[kb][8], sc[kb][9], sc[kb][10], sc[kb][11],
                             sc[kb][12], sc[kb][13], sc[kb][14], sc[kb][15]});
    }
    // O^T += V^T P^T: the D/32 output blocks are independent accumulators,
    // cycled in the inner loop; V^T fragments come from the row-major V tile
    // through the transposing read, one step ahead.
    {
      const uint16_t* vt = Vs[cur];
      constexpr int KS = kBN / 16;  // 16-key reduction steps per tile
      auto vfrag = [&](int ks, int db) -> bf16x8 {
        if constexpr (VCOPY)
          return lds_frag(vt + (db * 32 + l32) * VtStage::TSTR + ks * 16 + hh * 8);
        else
          return sw.tr(vt, ks * 16, db);
      };
      bf16x8 vf[2][D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vf[0][db] = vfrag(0, db);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) vf[(ks + 1) & 1][db] = vfrag(ks + 1, db);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = mfma32x32x16(vf[ks & 1][db], pb[ks >> 1][ks & 1], o[db]);
      }
    }
  };

  // Tile n+1 must have landed before the barrier that ends step n; the
  // loads of later tiles may stay in flight.
  const int loads_per_tile = (VCOPY ? 1 : 2) * TileStage::count(wave);
  auto step = [&](int n, auto mask_tag) {
    if (n + NBUF - 1 < ntiles) load_tile(n + NBUF - 1);
    compute(n, mask_tag);
    if constexpr (VCOPY) {
      if (n + 1 < ntiles) vts.store(tid, Vs[(n + 1) % NBUF]);
      wait_vmem_all();
    } else {
      wait_vmcnt_dyn(loads_per_tile * (min(n + NBUF - 1, ntiles - 1) - (n + 1)));
    }
    __syncthreads();
  };

#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < ntiles) load_tile(t);
  if constexpr (VCOPY) {
    vts.store(tid, Vs[0]);
    wait_vmem_all();
  } else {
    wait_vmcnt_dyn(loads_per_tile * (min(NBUF - 2, ntiles - 1)));
  }
  __syncthreads();

  // Tiles whose keys all precede this wave's first row need no mask; the
  // rest (the diagonal, and for the lower waves of the tile one tile wholly
  // above them, which the mask zeroes) do.  Every wave runs ntiles steps, so
  // the barriers match.
  const int n_full = min(ntiles, (wave_q0 + 1) / kBN);
  for (int n = 0; n < n_full; ++n) step(n, std::false_type{});
  for (int n = n_full; n < ntiles; ++n) step(n, std::true_type{});

  // ---- epilogue: normalise, write O and LSE at the original position ----
  const float lt = half_sum(l_run);
  const float inv = 1.f / lt;
  if (qvalid) {
    uint16_t* op = a.out + qoff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + r4 * 8 + hh * 4;
        st8(op + d, cvt4_bits(o[db][r4 * 4] * inv, o[db][r4 * 4 + 1] * inv,
                              o[db][r4 * 4 + 2] * inv, o[db][r4 * 4 + 3] * inv));
      }
    if (hh == 0 && a.lse != nullptr)
      a.lse[((long long)b * s.H + h) * s.N + qpos] = (m_run + __log2f(lt)) * kLn2;
  }
}

#ifndef S2A_FWD_WAVES_LARGE
#define S2A_FWD_WAVES_LARGE 4  // waves per workgroup for groups longer than 1024
#endif
#ifndef S2A_FWD_VCOPY
#define S2A_FWD_VCOPY 0  // V through a VGPR transposed copy (1) or transposing reads (0)
#endif

template <int D, int NW, bool ROPE>
hipError_t launch_fwd_t(FwdArgs a, const RopeTable* rope, hipStream_t stream) {
  constexpr int BM = NW * 32;
  a.tiles = (a.s.G + BM - 1) / BM;
  const long long grid = (long long)a.s.B * a.s.H * a.s.NG * a.tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  RopeTable rt{};
  if (ROPE) rt = *rope;
  hipLaunchKernelGGL((fwd_kernel<D, NW, ROPE, S2A_FWD_VCOPY != 0>), dim3((unsigned)grid), dim3(NW * 64), 0, stream,
                     a, rt);
  return hipGetLastError();
}

template <int D, bool ROPE>
hipError_t launch_fwd_d(const FwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  if (a.s.G <= 64) return launch_fwd_t<D, 2, ROPE>(a, rope, stream);
  if (a.s.G <= 1024) return launch_fwd_t<D, 4, ROPE>(a, rope, stream);
  return launch_fwd_t<D, S2A_FWD_WAVES_LARGE, ROPE>(a, rope, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  const bool r = rope != nullptr;
  if (a.s.D == 64) return r ? launch_fwd_d<64, true>(a, rope, stream) : launch_fwd_d<64, false>(a, rope, stream);
  return r ? launch_fwd_d<128, true>(a, rope, stream) : launch_fwd_d<128, false>(a, rope, stream);
}

}  // namespace s2a
