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
#ifndef S2A_FWD_VSTAGE
#define S2A_FWD_VSTAGE 1  // eight-wave workgroups stage K/V through VGPRs (1) or load straight into LDS (0)
#endif
constexpr float kLazy = 8.f;  // log2-domain slack before the softmax reference moves

// RB row blocks of 32 query rows per wave.  RB = 2 (one wave per SIMD, up to
// 512 registers) lets each K/V fragment read from LDS feed two MFMAs,
// halving the LDS traffic per FLOP; RB = 1 runs two waves per SIMD.
template <int D, int NW, int RB, bool ROPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RB == 2 ? 1 : 2, RB == 2 ? 1 : 2))) void fwd_kernel(FwdArgs a, RopeTable rope) {
  constexpr int BM = NW * 32 * RB;
  using TileStage = LdsStage<D, kBN, NW>;
  // Double-buffered K/V tiles (tile n in buffer n & 1), each buffer two
  // distinct LDS objects named at compile time: the compiler can then tell
  // the reads of one buffer from the loads filling the other and does not
  // make the reads wait for a tile still in flight.  Workgroups of 256 or
  // more rows stage K/V through VGPRs (VST): each thread loads its chunks of
  // tile n+1 at the start of step n and writes them to LDS at its end, which
  // on gfx950 competes far less with the step's LDS reads than
  // direct-to-LDS loads do.  Smaller workgroups load straight into LDS.
  constexpr bool VST = BM >= 256 && S2A_FWD_VSTAGE;
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[TileStage::ELEMS];
  auto kbuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(c)::value) return Ks1; else return Ks0;
  };
  auto vbuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(c)::value) return Vs1; else return Vs0;
  };
  using P0 = std::false_type;
  using P1 = std::true_type;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const TileLane<D> sw(lane);
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

  // ---- this lane's query rows (one per row block), held as MFMA B operands ----
  const int wave_q0 = t * BM + wave * 32 * RB;
  int qi[RB], qpos[RB];
  bool qvalid[RB];
  long long qoff[RB];
  // The softmax scale and log2(e) are folded into q once (one bf16
  // rounding of q * scale * log2 e), so S^T comes out of the MFMA in log2
  // units and P = exp2(S - m) needs no multiply.
  bf16x8 qf[RB][D / 16];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    qi[rb] = wave_q0 + rb * 32 + l32;
    qvalid[rb] = qi[rb] < s.G;
    qpos[rb] = qvalid[rb] ? orig_pos(base, qi[rb], s.N) : 0;
    qoff[rb] = ((long long)(b * (long long)s.N + qpos[rb]) * s.H + h) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4 raw = qvalid[rb] ? ld16(a.q + qoff[rb] + kk * 16 + hh * 8) : zero_u4();
      float x[8];
      unpack8(raw, x);
      if constexpr (ROPE) rope_rotate8(x, qpos[rb], rope.rev, kk * 16 + hh * 8, false);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= a.scale_log2;
      qf[rb][kk] = as_bf16x8(pack8(x));
    }
  }

  f32x16 o[RB][D / 32];
  // Softmax reference m_run (log2 units, -inf before the first tile).  The
  // S^T accumulators start at s0 = -m_run (0 before the first tile), so the
  // MFMA hands back S - m_run and P = exp2 of it.
  float m_run[RB], l_run[RB];  // l_run: this lane's half of the running row sum
  f32x16 s0[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[rb][i] = zero16();
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
    s0[rb] = zero16();
  }

  const int rows_end = min((t + 1) * BM, s.G);
  const int ntiles = (rows_end + kBN - 1) / kBN;

  const TileStage ts(wave, lane, (int)kv_row);
  // K and V tiles go straight from global memory into the padded LDS tiles;
  // rows past the group end point at the group's last row (their keys are
  // masked, so the values never contribute).
  auto load_tile = [&](int n, auto c) __attribute__((always_inline)) {
    const int key0 = n * kBN;
    const uint16_t* kt = contig_tile(kb_ptr, kv_row, base, key0, kBN, s.G, s.N);
    if (kt != nullptr) {
      ts.load_contig(kt, kbuf(c), wave);
      ts.load_contig(vb_ptr + (kt - kb_ptr), vbuf(c), wave);
    } else {
      auto rows = [&](const uint16_t* head0) {
        return [=, &s](int row) {
          const int j = min(key0 + row, s.G - 1);
          return head0 + orig_pos(base, j, s.N) * kv_row;
        };
      };
      ts.load_rows(rows(kb_ptr), kbuf(c), wave, lane);
      ts.load_rows(rows(vb_ptr), vbuf(c), wave, lane);
    }
  };

  // Tiles whose keys all precede this wave's first row need no mask; the
  // rest (the diagonal, and for the lower row blocks one tile wholly above
  // them, which the mask zeroes) do.
  const int n_full = min(ntiles, (wave_q0 + 1) / kBN);

  // One k/v tile: S^T = K Q^T, online softmax, O^T += V^T P^T for each row
  // block.  MASK only for the tiles from n_full on.
  auto compute = [&](int n, auto mask_tag, auto c) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int NB = kBN / 32;  // 32-key blocks per tile
    const int key0 = n * kBN;
    // S^T: each K fragment (one per 32-key block and k-step) is read once
    // and feeds one MFMA per row block; the 2*RB accumulators are
    // independent, so back-to-back MFMAs never wait on each other.
    f32x16 sc[RB][NB];
    {
      const uint16_t* kt = kbuf(c);
      constexpr int KD = 3;  // K fragments in flight: reads run two k-steps ahead
      bf16x8 kf[KD][NB];
#pragma unroll
      for (int kk = 0; kk < KD - 1; ++kk)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) kf[kk][kb] = sw.row(kt, kb * 32, kk);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + KD - 1 < D / 16) {
#pragma unroll
          for (int kb = 0; kb < NB; ++kb) kf[(kk + KD - 1) % KD][kb] = sw.row(kt, kb * 32, kk + KD - 1);
        }
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            sc[rb][kb] = mfma32x32x16(kf[kk % KD][kb], qf[rb][kk], kk == 0 ? s0[rb] : sc[rb][kb]);
      }
      // Keep the K reads (KD-1) k-steps ahead of the MFMAs that use them:
      // the scheduler would otherwise sink each read next to its use and
      // expose the LDS latency.
      __builtin_amdgcn_sched_group_barrier(0x100, (KD - 1) * NB, 0);
#pragma unroll
      for (int i = 0; i < (D / 16) * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
        if (i < (D / 16 - (KD - 1)) * NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    bf16x8 pb[RB][NB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (MASK) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = key0 + kb * 32 + acc_row(r, hh);
            if (j > qi[rb]) sc[rb][kb][r] = -INFINITY;
          }
      }
      // Online softmax in the exp2 domain with a lazily moved reference: the
      // reference moves (and O, l are rescaled) only when some row's max
      // exceeds it by more than kLazy (so p <= 2^kLazy), and on the first
      // tile; otherwise the stale reference stays, which changes nothing in
      // exact arithmetic.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[rb][kb][r]);
      mx = half_max(mx);  // relative to m_run (absolute before the first tile)
      const bool first = m_run[rb] == -INFINITY;
      if (__any(mx > kLazy || first)) {
        float m_new = first ? mx : m_run[rb] + fmaxf(mx, 0.f);
        if (mx == -INFINITY) m_new = m_run[rb];  // nothing visible yet
        const float alpha = m_new == m_run[rb] ? 1.f : fast_exp2(m_run[rb] - m_new);
        const float shift = m_new == -INFINITY ? 0.f : m_new - (first ? 0.f : m_run[rb]);
        m_run[rb] = m_new;
        l_run[rb] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[rb][i] *= alpha;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[rb][kb][r] -= shift;
        const float neg = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
#pragma unroll
        for (int r = 0; r < 16; ++r) s0[rb][r] = neg;
      }
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(sc[rb][kb][r]);
          sc[rb][kb][r] = pv;
          rs += pv;
        }
      l_run[rb] += rs;
      // P as bf16 B operands: accumulator elements 0..7 and 8..15 of each
      // 32-key block are the two 16-key halves of the reduction.
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        pb[rb][kb][0] = cvt8(f32x8{sc[rb][kb][0], sc[rb][kb][1], sc[rb][kb][2], sc[rb][kb][3],
                                   sc[rb][kb][4], sc[rb][kb][5], sc[rb][kb][6], sc[rb][kb][7]});
        pb[rb][kb][1] = cvt8(f32x8{sc[rb][kb][8], sc[rb][kb][9], sc[rb][kb][10], sc[rb][kb][11],
                                   sc[rb][kb][12], sc[rb][kb][13], sc[rb][kb][14], sc[rb][kb][15]});
      }
    }
    // O^T += V^T P^T: each V^T fragment (read through the transposing read
    // from the row-major V tile, one step ahead) feeds one MFMA per row
    // block; the D/32 * RB output blocks are independent accumulators.
    {
      const uint16_t* vt = vbuf(c);
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
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            o[rb][db] = mfma32x32x16(vf[ks & 1][db], pb[rb][ks >> 1][ks & 1], o[rb][db]);
      }
    }
  };

  // VGPR staging (VST): thread tid owns 16-byte chunks tid, tid + NW*64, ...
  // of the K tile followed by the V tile (chunk = tile row * D/8 + column
  // chunk).  A contiguous tile needs one 64-bit add per chunk.
  constexpr int kCh = D / 8;
  constexpr int kThreads = NW * 64;
  constexpr int kPer = VST ? 2 * kBN * kCh / kThreads : 1;
  static_assert(!VST || (2 * kBN * kCh) % kThreads == 0, "whole chunks per thread");
  u32x4 stg[kPer];
  auto chunk = [&](int i, int& tensor, int& row, int& col) __attribute__((always_inline)) {
    const int item = tid + i * kThreads;
    tensor = item / (kBN * kCh);
    const int rem = item - tensor * (kBN * kCh);
    row = rem / kCh;
    col = (rem % kCh) * 8;
  };
  auto gload_tile = [&](int n) __attribute__((always_inline)) {
    const int key0 = n * kBN;
    const uint16_t* kt = contig_tile(kb_ptr, kv_row, base, key0, kBN, s.G, s.N);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int tensor, row, col;
      chunk(i, tensor, row, col);
      const uint16_t* head0 = tensor ? vb_ptr : kb_ptr;
      const uint16_t* src;
      if (kt != nullptr)
        src = head0 + (kt - kb_ptr) + row * kv_row + col;
      else
        src = head0 + orig_pos(base, min(key0 + row, s.G - 1), s.N) * kv_row + col;
      stg[i] = ld16(src);
    }
  };
  auto swrite_tile = [&](auto c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int tensor, row, col;
      chunk(i, tensor, row, col);
      st16((tensor ? vbuf(c) : kbuf(c)) + row * (D + 8) + col, stg[i]);
    }
  };

  // Step n (buffer n & 1): start loading tile n+1 (into the other buffer,
  // or into VGPRs written to it at the end), compute tile n, wait for tile
  // n+1 and meet at the barrier.  Every wave runs ntiles steps, so the
  // barriers match.
  auto step = [&](int n, auto mask_tag, auto c) __attribute__((always_inline)) {
    using Next = std::integral_constant<bool, !decltype(c)::value>;
    if constexpr (VST) {
      if (n + 1 < ntiles) gload_tile(n + 1);
      compute(n, mask_tag, c);
      if (n + 1 < ntiles) swrite_tile(Next{});
    } else {
      if (n + 1 < ntiles) load_tile(n + 1, Next{});
      compute(n, mask_tag, c);
      wait_vmem_all();
    }
    lds_barrier();
  };
  // Steps n .. n1-1, unrolled by two so each names its buffer statically.
  auto run = [&](int n, int n1, auto mask_tag) __attribute__((always_inline)) {
    if (n < n1 && (n & 1)) step(n++, mask_tag, P1{});
    for (; n + 1 < n1; n += 2) {
      step(n, mask_tag, P0{});
      step(n + 1, mask_tag, P1{});
    }
    if (n < n1) step(n, mask_tag, P0{});
  };

  if constexpr (VST) {
    gload_tile(0);
    swrite_tile(P0{});
  } else {
    load_tile(0, P0{});
    wait_vmem_all();
  }
  lds_barrier();
  run(0, n_full, std::false_type{});
  run(n_full, ntiles, std::true_type{});

  // ---- epilogue: normalise, write O and LSE at the original position ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lt = half_sum(l_run[rb]);
    const float inv = 1.f / lt;
    if (qvalid[rb]) {
      uint16_t* op = a.out + qoff[rb];
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = db * 32 + r4 * 8 + hh * 4;
          st8(op + d, cvt4_bits(o[rb][db][r4 * 4] * inv, o[rb][db][r4 * 4 + 1] * inv,
                                o[rb][db][r4 * 4 + 2] * inv, o[rb][db][r4 * 4 + 3] * inv));
        }
      if (hh == 0 && a.lse != nullptr)
        a.lse[((long long)b * s.H + h) * s.N + qpos[rb]] = (m_run[rb] + __log2f(lt)) * kLn2;
    }
  }
}

#ifndef S2A_FWD_BIG
#define S2A_FWD_BIG 0  // groups longer than 1024: 4 waves x 64 rows (1) or 8 waves x 32 rows (0)
#endif

template <int D, int NW, int RB, bool ROPE>
hipError_t launch_fwd_t(FwdArgs a, const RopeTable* rope, hipStream_t stream) {
  constexpr int BM = NW * 32 * RB;
  a.tiles = (a.s.G + BM - 1) / BM;
  const long long grid = (long long)a.s.B * a.s.H * a.s.NG * a.tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  RopeTable rt{};
  if (ROPE) rt = *rope;
  hipLaunchKernelGGL((fwd_kernel<D, NW, RB, ROPE>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a, rt);
  return hipGetLastError();
}

template <int D, bool ROPE>
hipError_t launch_fwd_d(const FwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  if (a.s.G <= 64) return launch_fwd_t<D, 2, 1, ROPE>(a, rope, stream);
  if (a.s.G <= 1024) return launch_fwd_t<D, 4, 1, ROPE>(a, rope, stream);
  if constexpr (S2A_FWD_BIG) return launch_fwd_t<D, 4, 2, ROPE>(a, rope, stream);
  return launch_fwd_t<D, 8, 1, ROPE>(a, rope, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  const bool r = rope != nullptr;
  if (a.s.D == 64) return r ? launch_fwd_d<64, true>(a, rope, stream) : launch_fwd_d<64, false>(a, rope, stream);
  return r ? launch_fwd_d<128, true>(a, rope, stream) : launch_fwd_d<128, false>(a, rope, stream);
}

}  // namespace s2a
