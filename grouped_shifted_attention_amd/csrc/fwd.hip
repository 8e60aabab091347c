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

template <int D, int NW, bool ROPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(FwdArgs a, RopeTable rope) {
  constexpr int BM = NW * 32;
  using TileStage = LdsStage<D, kBN, NW>;
  // Double-buffered K/V tiles as four distinct LDS objects, each chosen at
  // compile time (tile n lives in buffer n & 1): the compiler can then tell
  // the reads of the current tile from the direct loads filling the other
  // buffer, and does not make the reads wait for the tile still in flight.
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[kBN * D];
  auto kbuf = [&](auto p) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(p)::value) return Ks1; else return Ks0;
  };
  auto vbuf = [&](auto p) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(p)::value) return Vs1; else return Vs0;
  };
  using P0 = std::false_type;
  using P1 = std::true_type;

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
  auto load_tile = [&](int n, auto p) __attribute__((always_inline)) {
    const int key0 = n * kBN;
    const uint16_t* kt = contig_tile(kb_ptr, kv_row, base, key0, kBN, s.G, s.N);
    if (kt != nullptr) {
      ts.load_contig(kt, kbuf(p), wave);
      ts.load_contig(vb_ptr + (kt - kb_ptr), vbuf(p), wave);
    } else {
      auto rows = [&](const uint16_t* head0) {
        return [=, &s](int row) {
          const int j = min(key0 + row, s.G - 1);
          return head0 + orig_pos(base, j, s.N) * kv_row;
        };
      };
      ts.load_rows(rows(kb_ptr), kbuf(p), wave, lane);
      ts.load_rows(rows(vb_ptr), vbuf(p), wave, lane);
    }
  };

  // One k/v tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  MASK is set
  // only for tiles that reach past this wave's first row (the diagonal).
  auto compute = [&](int n, auto mask_tag, auto p) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int key0 = n * kBN;
    // S^T: the two 32-key blocks are independent accumulators, interleaved
    // so back-to-back MFMAs never wait on each other; K fragments are read
    // from LDS one k-step ahead.
    f32x16 sc[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) sc[kb] = zero16();
    {
      const uint16_t* kt = kbuf(p);
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
      const uint16_t* vt = vbuf(p);
      constexpr int KS = kBN / 16;  // 16-key reduction steps per tile
      bf16x8 vf[2][D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vf[0][db] = sw.tr(vt, 0, db);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) vf[(ks + 1) & 1][db] = sw.tr(vt, (ks + 1) * 16, db);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = mfma32x32x16(vf[ks & 1][db], pb[ks >> 1][ks & 1], o[db]);
      }
    }
  };

  // Step n: start loading tile n+1 into the other buffer, compute tile n,
  // then wait for tile n+1 and meet at the barrier (after which buffer n & 1
  // may be overwritten).
  auto step = [&](int n, auto mask_tag, auto p) __attribute__((always_inline)) {
    if (n + 1 < ntiles) load_tile(n + 1, std::integral_constant<bool, !decltype(p)::value>{});
    compute(n, mask_tag, p);
    wait_vmem_all();
    lds_barrier();
  };
  // Steps n0 .. n1-1, unrolled by two so each names its buffer statically.
  auto run = [&](int n, int n1, auto mask_tag) __attribute__((always_inline)) {
    if (n < n1 && (n & 1)) step(n++, mask_tag, P1{});
    for (; n + 1 < n1; n += 2) {
      step(n, mask_tag, P0{});
      step(n + 1, mask_tag, P1{});
    }
    if (n < n1) step(n, mask_tag, P0{});
  };

  load_tile(0, P0{});
  wait_vmem_all();
  lds_barrier();

  // Tiles whose keys all precede this wave's first row need no mask; the
  // rest (the diagonal, and for the lower waves of the tile one tile wholly
  // above them, which the mask zeroes) do.  Every wave runs ntiles steps, so
  // the barriers match.
  const int n_full = min(ntiles, (wave_q0 + 1) / kBN);
  run(0, n_full, std::false_type{});
  run(n_full, ntiles, std::true_type{});

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

template <int D, int NW, bool ROPE>
hipError_t launch_fwd_t(FwdArgs a, const RopeTable* rope, hipStream_t stream) {
  constexpr int BM = NW * 32;
  a.tiles = (a.s.G + BM - 1) / BM;
  const long long grid = (long long)a.s.B * a.s.H * a.s.NG * a.tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  RopeTable rt{};
  if (ROPE) rt = *rope;
  hipLaunchKernelGGL((fwd_kernel<D, NW, ROPE>), dim3((unsigned)grid), dim3(NW * 64), 0, stream,
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
