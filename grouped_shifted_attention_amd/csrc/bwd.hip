// S2-Attn backward kernels for gfx950.
//
// The pages give no backward pass; this is the calculus of the forward
// definition (AIMech "LongLoRA and Shifted Sparse Attention (S^2-Attn)",
// opening definition), recomputing P from the saved log-sum-exp:
//   P = exp(S - lse),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - Delta),  dQ = c dS K,  dK = c dS^T Q,   c = 1/sqrt(D)
// per group of rolled rows.  The S accumulators start at -lse*log2(e) and
// take one operand pre-scaled by c*log2(e) (one bf16 rounding), and the dP
// accumulators start at -Delta (both from the preprocess pass), so that
// P = exp2(acc) and dS = P * acc.  Rows and keys are addressed at their original
// positions (the roll by -shift and its inverse folded into indices), so dQ,
// dK, dV land where the forward read q, k, v.
//
// Two kernels, no atomics (bitwise deterministic):
//   dkdv_kernel  one workgroup per (batch, k/v head, group, 128-key tile);
//                each wave owns 32 keys, keeps K and V as MFMA B operands in
//                VGPRs and accumulates dK^T, dV^T over every q head sharing
//                the k/v head and every 32-row q step from the diagonal to
//                the group end.  4 MFMA products per step; Q^T and dO^T are
//                read transposed (ds_read_b64_tr_b16) from row-major tiles.
//   dq_kernel    one workgroup per (batch, q head, group, q tile); each wave
//                owns 32 query rows and walks the k/v tiles up to the
//                diagonal.  3 MFMA products per tile.
#include "device_common.hpp"
#include "kernels.hpp"
#include "staging.hpp"

#include <type_traits>

namespace s2a {

namespace {

constexpr int kBN = 64;  // dq_kernel: keys per k/v tile

// Inverse RoPE rotation of one lane's accumulator block before the store:
// elements 4*r4 .. 4*r4+3 hold columns d0 .. d0+3, two adjacent pairs.
__device__ __forceinline__ void rope_unrotate4(float x[4], int pos, const double* rev, int d0) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const double r = (double)pos * rev[(d0 >> 1) + e];
    float sn, cs;
    sincos_turns((float)(r - floor(r)), sn, cs);
    const float a = x[2 * e], b = x[2 * e + 1];
    x[2 * e] = a * cs + b * sn;
    x[2 * e + 1] = -a * sn + b * cs;
  }
}

// Scale, optionally un-rotate, round and store a C-layout accumulator whose
// lane holds one row (at `row_ptr`) and whose elements run over D.
template <int D, bool ROPE>
__device__ __forceinline__ void store_row_acc(uint16_t* row_ptr, const f32x16* acc, float scale, int hh, int pos,
                                              const RopeTable& rope) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = db * 32 + r4 * 8 + hh * 4;
      float x[4] = {acc[db][r4 * 4] * scale, acc[db][r4 * 4 + 1] * scale, acc[db][r4 * 4 + 2] * scale,
                    acc[db][r4 * 4 + 3] * scale};
      if constexpr (ROPE) rope_unrotate4(x, pos, rope.rev, d);
      st8(row_ptr + d, cvt4_bits(x[0], x[1], x[2], x[3]));
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int NW, bool ROPE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(BwdArgs a,
                                                                                                 RopeTable rope) {
  constexpr int BM = NW * 32;
  using TileStage = LdsStage<D, kBN, NW>;  // K rows (S^T; read transposed for dQ^T), V rows (dP^T)
  // Double-buffered K/V tiles as distinct LDS objects named at compile time
  // (tile n in buffer n & 1), so reads of one buffer never wait for the
  // direct loads into the other.
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[TileStage::ELEMS];
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
  const TileLane<D> sw(lane);
  const Shape& s = a.s;

  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int unit = logical / a.tiles;
  const int t = a.tiles - 1 - (logical - unit * a.tiles);
  const QUnit uq = decode_q_unit(unit, s);
  const int g = uq.g, h = uq.h, b = uq.b;
  const int sh = head_shift(h, s);
  const int kvh = h / (s.H / s.Hkv);
  const int base = g * s.G + sh;
  const long long kv_row = (long long)s.Hkv * D;
  const uint16_t* kb_ptr = a.k + (long long)b * s.N * kv_row + (long long)kvh * D;
  const uint16_t* vb_ptr = a.v + (long long)b * s.N * kv_row + (long long)kvh * D;

  const int wave_q0 = t * BM + wave * 32;
  const int qi = wave_q0 + l32;
  const bool qvalid = qi < s.G;
  const int qpos = qvalid ? orig_pos(base, qi, s.N) : 0;
  const long long qoff = ((long long)(b * (long long)s.N + qpos) * s.H + h) * D;
  // The q operand is q * c * log2(e) rounded to bf16 once (the forward's
  // rounding of it), so S comes out in log2 units.  Without RoPE it is
  // formed here from the caller's q; with RoPE the rotate pass formed it.
  bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 qw = qvalid ? ld16(a.q + qoff + kk * 16 + hh * 8) : zero_u4();
    if constexpr (!ROPE) qw = scale_bf16x8(qw, a.scale_log2);
    asm volatile("" : "+v"(qw));  // keep the fragment resident from here on
    qf[kk] = as_bf16x8(qw);
    dof[kk] = as_bf16x8(qvalid ? ld16(a.dout + qoff + kk * 16 + hh * 8) : zero_u4());
  }
  const long long stat_off = ((long long)b * s.H + h) * s.N + qpos;
  // Accumulator start values: every element of a lane belongs to its row.
  f32x16 s_init, dp_init;
  {
    const float nl = qvalid ? a.nlse2[stat_off] : 0.f;
    const float nd = qvalid ? a.ndelta[stat_off] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s_init[r] = nl;
      dp_init[r] = nd;
    }
  }

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = zero16();

  const int rows_end = min((t + 1) * BM, s.G);
  const int ntiles = (rows_end + kBN - 1) / kBN;

  const TileStage ts(wave, lane, (int)kv_row);
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

  auto compute = [&](int n, auto mask_tag, auto p) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* kt = kbuf(p);
    const uint16_t* vt = vbuf(p);
    const int key0 = n * kBN;
    // Two 32-key halves in turn (keeps the live S/dP set small enough for
    // two waves per SIMD).  Per half: S^T = K Q^T and dP^T = V dO^T (two
    // accumulators, K/V fragments read one k-step ahead), P and dS on the
    // VALU, then dQ^T += K^T dS^T with K^T read transposed from the
    // row-major K tile.
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      // A masked half whose keys all follow this wave's last row adds exact
      // zeros to dQ: skip it (the workgroup's later waves need those keys).
      if constexpr (MASK) {
        if (key0 + kb * 32 > wave_q0 + 31) continue;
      }
      f32x16 sc, dp;
      {
        bf16x8 kf[2], vf[2];
        kf[0] = sw.row(kt, kb * 32, 0);
        vf[0] = sw.row(vt, kb * 32, 0);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk + 1 < D / 16) {
            kf[(kk + 1) & 1] = sw.row(kt, kb * 32, kk + 1);
            vf[(kk + 1) & 1] = sw.row(vt, kb * 32, kk + 1);
          }
          sc = mfma32x32x16(kf[kk & 1], qf[kk], kk == 0 ? s_init : sc);
          dp = mfma32x32x16(vf[kk & 1], dof[kk], kk == 0 ? dp_init : dp);
        }
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(sc[r]);
        if constexpr (MASK) {
          const int j = key0 + kb * 32 + acc_row(r, hh);
          if (j > qi) p = 0.f;
        }
        ds[r] = p * dp[r];
      }
      bf16x8 dsb[2];
      dsb[0] = cvt8(f32x8{ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]});
      dsb[1] = cvt8(f32x8{ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]});
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 tf[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) tf[db] = sw.tr(kt, kb * 32 + hf * 16, db);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = mfma32x32x16(tf[db], dsb[hf], dq[db]);
      }
    }
  };

  // K/V tile walk: up from key 0 or down from the diagonal, alternating
  // between consecutive units when a unit's workgroups fit on one XCD's CUs,
  // so that they, which then either start together or end together, stay on
  // the same k/v tile in L2 (as in the forward kernel).
  const bool walk_down = a.tiles <= kCusPerXcd && (unit & 1) != 0;
  auto tile_at = [&](int i) __attribute__((always_inline)) { return walk_down ? ntiles - 1 - i : i; };

  // Step i: load the tile of step i+1 into the other buffer, compute the tile
  // of step i, wait for the load, barrier.  Unrolled by two so each step
  // names its buffer.
  auto step = [&](int n, auto mask_tag, auto p) __attribute__((always_inline)) {
    if (n + 1 < ntiles) load_tile(tile_at(n + 1), std::integral_constant<bool, !decltype(p)::value>{});
    compute(tile_at(n), mask_tag, p);
    wait_vmem_all();
    lds_barrier();
  };
  auto run = [&](int n, int n1, auto mask_tag) __attribute__((always_inline)) {
    if (n < n1 && (n & 1)) step(n++, mask_tag, P1{});
    for (; n + 1 < n1; n += 2) {
      step(n, mask_tag, P0{});
      step(n + 1, mask_tag, P1{});
    }
    if (n < n1) step(n, mask_tag, P0{});
  };

  load_tile(tile_at(0), P0{});
  wait_vmem_all();
  lds_barrier();

  // Tiles before n_full lie wholly left of this wave's diagonal and need no
  // mask; walking up they come first, walking down last.
  const int n_full = min(ntiles, (wave_q0 + 1) / kBN);
  if (walk_down) {
    run(0, ntiles - n_full, std::true_type{});
    run(ntiles - n_full, ntiles, std::false_type{});
  } else {
    run(0, n_full, std::false_type{});
    run(n_full, ntiles, std::true_type{});
  }

  if (qvalid) store_row_acc<D, ROPE>(a.dq + qoff, dq, a.scale, hh, qpos, rope);
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
// Eight waves per workgroup, two per SIMD, specialised in pairs that share
// 32 keys: the "P wave" (waves 0-3) computes S = Q K^T, P and dV^T += dO^T P
// and publishes its bf16 P through LDS; the "dS wave" (waves 4-7) runs one
// step behind on the same keys and computes dP = dO V^T, dS = P (dP - Delta)
// and dK^T += Q^T dS.  Each keeps one of K/V and one of dK/dV, which halves
// the registers a wave needs against one wave doing all four products.
// q/dout tiles sit in a 6-deep LDS ring and the dS wave runs two steps
// behind the P wave, so the waves meet at a barrier only every second step:
// in the two steps between barriers the P waves read steps n, n+1, the dS
// waves steps n-2, n-1, and steps n+2, n+3 are written.  The rows' lse and
// Delta ride along at the end of the dout tile; P travels through four LDS
// slots (step & 3) as fp16, whose 11-bit significand keeps dS = P (dP -
// Delta) from inheriting the 8-bit rounding of the bf16 P that feeds dV (P
// lies in [0, 1], where fp16 is exact to 2^-11 relative down to 2^-14 and
// to 2^-25 absolute below).
//
// The largest P and dS of a key sit in the rows just past it: the masked
// (diagonal) step.  There the dV and dK products take their bf16 operand as
// hi + lo (two MFMAs each), so their rounding error, which would otherwise
// dominate the k/v gradients summed over grouped-query heads, drops to that
// of an fp32 operand.  Masked steps are about one in G/128 per head.
constexpr int kDkdvPairs = 4;
constexpr int kDkdvWaves = 2 * kDkdvPairs;
constexpr int kBNK = kDkdvPairs * 32;  // keys per workgroup
constexpr int kBMQ = 32;               // q rows per step
constexpr int kStages = 6;

template <int D, bool ROPE>
__global__ __launch_bounds__(kDkdvWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_kernel(
    BwdArgs a, RopeTable rope) {
  using TileStage = LdsStage<D, kBMQ, kDkdvWaves>;
  // The ring's q and dout tiles are twelve distinct LDS objects, each named
  // at compile time (step m in stage m % 6).
  __shared__ __attribute__((aligned(16))) uint16_t Q0[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q2[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q3[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q4[TileStage::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Q5[TileStage::ELEMS];
  // dout tile, then the step's 32 lse values and 32 Delta values (fp32).
  constexpr int kOElems = TileStage::ELEMS + 2 * kBMQ * 2;
  __shared__ __attribute__((aligned(16))) uint16_t O0[kOElems];
  __shared__ __attribute__((aligned(16))) uint16_t O1[kOElems];
  __shared__ __attribute__((aligned(16))) uint16_t O2[kOElems];
  __shared__ __attribute__((aligned(16))) uint16_t O3[kOElems];
  __shared__ __attribute__((aligned(16))) uint16_t O4[kOElems];
  __shared__ __attribute__((aligned(16))) uint16_t O5[kOElems];
  auto qbuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    constexpr int C = decltype(c)::value;
    if constexpr (C == 0) return Q0; else if constexpr (C == 1) return Q1;
    else if constexpr (C == 2) return Q2; else if constexpr (C == 3) return Q3;
    else if constexpr (C == 4) return Q4; else return Q5;
  };
  auto obuf = [&](auto c) __attribute__((always_inline)) -> uint16_t* {
    constexpr int C = decltype(c)::value;
    if constexpr (C == 0) return O0; else if constexpr (C == 1) return O1;
    else if constexpr (C == 2) return O2; else if constexpr (C == 3) return O3;
    else if constexpr (C == 4) return O4; else return O5;
  };
  static_assert(kStages == 6, "the ring is unrolled by six");
  // P hand-over: [slot][pair][half][lane] 16 bytes (8 fp16); step m in slot m & 3.
  __shared__ __attribute__((aligned(16))) u32x4 Pbuf[4][kDkdvPairs][2][64];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const TileLane<D> sw(lane);
  const bool ds_wave = wave >= kDkdvPairs;
  const int pair = wave & (kDkdvPairs - 1);
  const Shape& s = a.s;

  // Work item: (b, kv head, group) units, key tiles with the most rows first.
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int unit = logical / a.tiles;
  const int tk = logical - unit * a.tiles;
  const int g = unit % s.NG;
  const int bk = unit / s.NG;
  const int kvh = bk % s.Hkv;
  const int b = bk / s.Hkv;
  const int rq = s.H / s.Hkv;  // q heads per k/v head
  const int h0 = kvh * rq;
  const int sh = head_shift(h0, s);  // shared by all rq q heads
  const int base = g * s.G + sh;
  const long long kv_row = (long long)s.Hkv * D;
  const long long q_row = (long long)s.H * D;

  // This lane's key; the P wave holds K, the dS wave V, as MFMA B operands.
  const int key_start = tk * kBNK;
  const int kw0 = key_start + pair * 32;
  const int kj = kw0 + l32;
  const bool kvalid = kj < s.G;
  const int kpos = kvalid ? orig_pos(base, kj, s.N) : 0;
  const long long koff = ((long long)b * s.N + kpos) * kv_row + (long long)kvh * D;
  const uint16_t* kv_src = ds_wave ? a.v : a.k;
  bf16x8 kvf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kvf[kk] = as_bf16x8(kvalid ? ld16(kv_src + koff + kk * 16 + hh * 8) : zero_u4());


  f32x16 acc[D / 32];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = zero16();

  // Steps: every 32-row block from the first row that can see this tile's
  // keys to the group end x every q head sharing this k/v head.  The row
  // blocks go from the group end down (heads inner), so the workgroups of a
  // unit, which run side by side on one XCD and all start at the group end,
  // read the same q/dout tiles at the same time and share them in L2; each
  // stops at its own diagonal.  (Walking up from each diagonal, head by
  // head, put them on different heads within a few steps: under 8:1
  // grouped-query sharing a unit's q/dout rows do not fit in L2, and the
  // kernel read 25x its algorithmic bytes from HBM.)
  const int steps_per_head = (s.G - key_start + kBMQ - 1) / kBMQ;
  const int nsteps = steps_per_head * rq;

  const TileStage ts(wave, lane, (int)q_row);
  auto stats = [&](auto c) __attribute__((always_inline)) -> float* {
    return reinterpret_cast<float*>(obuf(c) + TileStage::ELEMS);
  };
  // Staging through VGPRs: thread tid owns 16-byte chunks tid,
  // tid + 512, ... of the step's q tile followed by its dout tile (chunk =
  // tile row * D/8 + column chunk); wave 0 also loads the rows' statistics
  // (lanes 0-31 -lse*log2 e, lanes 32-63 -Delta, slot m holding tile row
  // rowperm32(m)).  Two register sets (step m in set m & 1): the loads of
  // step n+3 are issued at the start of step n and written to LDS at the
  // end of step n+1, so they have two steps to arrive.
  constexpr int kCh = D / 8;
  constexpr int kChunks = kBMQ * kCh;  // per tensor
  constexpr int kThreads = kDkdvWaves * 64;
  static_assert(2 * kChunks % kThreads == 0, "whole chunks per thread");
  constexpr int kPer = 2 * kChunks / kThreads;
  u32x4 stg[2][kPer];
  float stg_stat[2] = {0.f, 0.f};
  // Steps are loaded in order; (ld_j, ld_hi) is the row block and q head of
  // the next one (running counts, no division per step).  Every interval
  // issues the same loads, also past the last step (those re-read the last
  // step's rows, still in L2, into stages nobody reads): with no branch
  // around them the compiler's wait before each LDS write counts only the
  // older register set, instead of waiting for the loads just issued as well.
  int ld_j = steps_per_head - 1, ld_hi = 0;
  auto gload_step = [&](auto set) __attribute__((always_inline)) {
    constexpr int R = decltype(set)::value;
    const bool past = ld_j < 0;
    const int hi = past ? rq - 1 : ld_hi, i0 = key_start + (past ? 0 : ld_j) * kBMQ;
    if (++ld_hi == rq) {
      ld_hi = 0;
      --ld_j;
    }
    const long long head_off = (long long)b * s.N * q_row + (long long)(h0 + hi) * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + i * kThreads;
      const int tensor = item / kChunks;
      const int rem = item - tensor * kChunks;
      const int row = min(i0 + rem / kCh, s.G - 1);
      stg[R][i] = ld16((tensor ? a.dout : a.q) + head_off + orig_pos(base, row, s.N) * q_row + (rem % kCh) * 8);
    }
    {  // every wave loads (equal load counts per wave); wave 0 writes
      const int i = min(i0 + rowperm32(l32), s.G - 1);
      const long long so = ((long long)b * s.H + h0 + hi) * s.N + orig_pos(base, i, s.N);
      stg_stat[R] = (hh ? a.ndelta : a.nlse2)[so];
    }
  };
  // Without RoPE the q chunks become the logit operand here: q * c * log2(e)
  // with one bf16 rounding, as the forward forms it.
  auto swrite_step = [&](auto c, auto set) __attribute__((always_inline)) {
    constexpr int R = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int item = tid + i * kThreads;
      const int tensor = item / kChunks;
      const int rem = item - tensor * kChunks;
      u32x4 w = stg[R][i];
      if constexpr (!ROPE) {
        if (tensor == 0) w = scale_bf16x8(w, a.scale_log2);
      }
      st16((tensor ? obuf(c) : qbuf(c)) + (rem / kCh) * (D + 8) + (rem % kCh) * 8, w);
    }
    if (wave == 0) stats(c)[lane] = stg_stat[R];
  };

  // Accumulator start values for a step: element r of the lane belongs to
  // row slot 8*(r/4) + 4*hh + r%4, whose statistic sits at that slot.
  auto row_stats = [&](const float* st) __attribute__((always_inline)) -> f32x16 {
    f32x16 v;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&st[8 * r4 + 4 * hh]);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * r4 + e] = x[e];
    }
    return v;
  };

  // acc += T K^T (or T V^T) for the step's 32-row tile T in LDS: one
  // dependent chain of D/16 MFMAs whose A fragments are read three k-steps
  // ahead (the compiler would otherwise put each read right before its MFMA
  // and expose the LDS latency at every k-step).
  auto chain_mfma = [&](f32x16& acc_, const uint16_t* t) __attribute__((always_inline)) {
    constexpr int kPF = 4;  // fragments in flight (4 timed best of 2, 3, 4, 6, 8)
    bf16x8 fa[kPF];
#pragma unroll
    for (int kk = 0; kk < kPF - 1; ++kk) fa[kk] = sw.row(t, 0, kk);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + kPF - 1 < D / 16) fa[(kk + kPF - 1) % kPF] = sw.row(t, 0, kk + kPF - 1);
      acc_ = mfma32x32x16(fa[kk % kPF], kvf[kk], acc_);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kPF - 1, 0);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (kk + kPF - 1 < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // P wave: S = Q K^T - lse (log2 units; lane column = key, elements = rows
  // 8*(r/4) + 4*hh + r%4 of the step), P = exp2(S), publish P,
  // dV^T += dO^T P.
  auto p_step = [&](int step, int i0, bool mask, auto c) __attribute__((always_inline)) {
    const uint16_t* qt = qbuf(c);
    const uint16_t* ot = obuf(c);
    const float* st = stats(c);
    f32x16 sc = row_stats(st);
    chain_mfma(sc, qt);
    // dO^T fragments of the dV product, read before the exp2 work that
    // needs the chain's result, so their LDS latency hides behind it.
    bf16x8 ofr[2][D / 32];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) ofr[hf][db] = sw.tr(ot, hf * 16, db);
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = fast_exp2(sc[r]);
    if (__builtin_expect(mask, 0)) {  // one uniform branch around the selects, none per element
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + acc_row(r, hh);
        p[r] = (kj > row || row >= s.G) ? 0.f : p[r];
      }
    }
    const f32x8 pf[2] = {f32x8{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]},
                         f32x8{p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]}};
    bf16x8 pb[2];
    pb[0] = cvt8(pf[0]);
    pb[1] = cvt8(pf[1]);
    Pbuf[step & 3][pair][0][lane] = __builtin_bit_cast(u32x4, __builtin_convertvector(pf[0], f16x8));
    Pbuf[step & 3][pair][1][lane] = __builtin_bit_cast(u32x4, __builtin_convertvector(pf[1], f16x8));
    // Raised issue priority over the closing products: when both waves of a
    // SIMD are ready, these MFMAs go first and the partner's VALU work fills
    // the gaps between them.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma32x32x16(ofr[hf][db], pb[hf], acc[db]);
    if (__builtin_expect(mask, 0)) {  // diagonal step: the part of P that bf16 missed
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8 pl = bf16_residual8(pf[hf], pb[hf]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma32x32x16(ofr[hf][db], pl, acc[db]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // dS wave (two steps behind): dP = dO V^T - Delta, dS = P dP with the P
  // wave's published P, dK^T += Q^T dS.
  auto ds_step = [&](int step, bool mask, auto c) __attribute__((always_inline)) {
    const uint16_t* qt = qbuf(c);
    const uint16_t* ot = obuf(c);
    const float* st = stats(c);
    f32x16 dp = row_stats(st + kBMQ);
    chain_mfma(dp, ot);
    // Q^T fragments of the dK product, read ahead of the dS work.
    bf16x8 qfr[2][D / 32];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) qfr[hf][db] = sw.tr(qt, hf * 16, db);
    const f16x8 ph0 = __builtin_bit_cast(f16x8, Pbuf[step & 3][pair][0][lane]);
    const f16x8 ph1 = __builtin_bit_cast(f16x8, Pbuf[step & 3][pair][1][lane]);
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = __builtin_fmaf((float)(r < 8 ? ph0[r] : ph1[r - 8]), dp[r], 0.f);  // v_fma_mix
    const f32x8 dsf[2] = {f32x8{ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]},
                          f32x8{ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]}};
    bf16x8 dsb[2];
    dsb[0] = cvt8(dsf[0]);
    dsb[1] = cvt8(dsf[1]);
    __builtin_amdgcn_s_setprio(1);  // as in the P wave
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] = mfma32x32x16(qfr[hf][db], dsb[hf], acc[db]);
    if (__builtin_expect(mask, 0)) {  // diagonal step: the part of dS that bf16 missed
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8 dl = bf16_residual8(dsf[hf], dsb[hf]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] = mfma32x32x16(qfr[hf][db], dl, acc[db]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Per q head: steps whose rows all precede this pair's keys contribute
  // nothing and are skipped; the step crossing the diagonal, and a last step
  // that runs past the group end, are masked.
  const int skip = min(steps_per_head, (kw0 - key_start) / kBMQ);
  const int diag_end = min(steps_per_head, (kw0 + 31 - key_start) / kBMQ + 1);
  const int ragged = ((s.G - key_start) % kBMQ) != 0 ? steps_per_head - 1 : steps_per_head;
  // j: a step's row block, counted from key_start.
  auto step_kind = [&](int j) __attribute__((always_inline)) {  // 0 skip, 1 masked, 2 full
    return j < skip ? 0 : ((j < diag_end || j >= ragged) ? 1 : 2);
  };
  int cur_j = steps_per_head - 1, cur_hi = 0;  // row block and q head of step n (P wave)
  int ds_j = steps_per_head - 1, ds_hi = 0;    // of step n - 2 (dS wave)

  using R0 = std::integral_constant<int, 0>;
  using R1 = std::integral_constant<int, 1>;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  gload_step(R0{});
  swrite_step(S0{}, R0{});
  gload_step(R1{});
  swrite_step(S1{}, R1{});
  gload_step(R0{});
  lds_barrier();

  // Step n (stage c = n % 6): the P wave does step n, the dS wave step n-2;
  // the loads of step n+3 are issued and step n+2 is written into the stage
  // that held step n-4.  A barrier follows every odd step, so between two
  // barriers (steps n, n+1 with n even) the reads touch steps n-2 .. n+1
  // and the writes steps n+2, n+3 (P slots n & 3, n+1 & 3; read two steps
  // later, across a barrier): six distinct stages, four distinct P slots.
  // nsteps+2 steps in all, identical for every wave.
  // The two roles run separate copies of the loop (the role is fixed per
  // wave), and every step runs the same instructions: steps that lie wholly
  // before this pair's keys are not skipped but fully masked (P = 0, so they
  // add exact zeros).  Without branches around the products the accumulators
  // keep their registers across steps instead of being copied at every join.
  auto iter = [&](int n, auto c, auto role) __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;
    constexpr bool DS = decltype(role)::value;
    gload_step(std::integral_constant<int, (C + 1) & 1>{});
    if constexpr (!DS) {
      if (n < nsteps) p_step(n, key_start + cur_j * kBMQ, step_kind(cur_j) != 2, c);
      if (++cur_hi == rq) {
        cur_hi = 0;
        --cur_j;
      }
    } else {
      if (n >= 2) {
        ds_step(n - 2, step_kind(ds_j) != 2, std::integral_constant<int, (C + 4) % 6>{});
        if (++ds_hi == rq) {
          ds_hi = 0;
          --ds_j;
        }
      }
    }
    swrite_step(std::integral_constant<int, (C + 2) % 6>{}, std::integral_constant<int, C & 1>{});
#ifdef S2A_DEBUG_BARRIERS
    lds_barrier();  // race-check build: a full barrier after every step
#else
    if constexpr ((C & 1) != 0) lds_barrier();
#endif
  };
  auto run = [&](auto role) __attribute__((always_inline)) {
    for (int n = 0; n <= nsteps + 1; n += 6) {
      iter(n, std::integral_constant<int, 0>{}, role);
      if (n + 1 <= nsteps + 1) iter(n + 1, std::integral_constant<int, 1>{}, role);
      if (n + 2 <= nsteps + 1) iter(n + 2, std::integral_constant<int, 2>{}, role);
      if (n + 3 <= nsteps + 1) iter(n + 3, std::integral_constant<int, 3>{}, role);
      if (n + 4 <= nsteps + 1) iter(n + 4, std::integral_constant<int, 4>{}, role);
      if (n + 5 <= nsteps + 1) iter(n + 5, std::integral_constant<int, 5>{}, role);
    }
  };
  if (ds_wave)
    run(std::true_type{});
  else
    run(std::false_type{});

  if (kvalid) {
    if (ds_wave)
      store_row_acc<D, ROPE>(a.dk + koff, acc, kLn2, hh, kpos, rope);  // q arrives scaled by c log2 e
    else
      store_row_acc<D, false>(a.dv + koff, acc, 1.f, hh, kpos, rope);
  }
}

template <int D, int NW, bool ROPE>
hipError_t launch_dq_t(BwdArgs a, const RopeTable* rope, hipStream_t stream) {
  constexpr int BM = NW * 32;
  a.tiles = (a.s.G + BM - 1) / BM;
  const long long grid = (long long)a.s.B * a.s.H * a.s.NG * a.tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  RopeTable rt{};
  if (ROPE) rt = *rope;
  hipLaunchKernelGGL((dq_kernel<D, NW, ROPE>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, a, rt);
  return hipGetLastError();
}

template <int D, bool ROPE>
hipError_t launch_dkdv_t(BwdArgs a, const RopeTable* rope, hipStream_t stream) {
  a.tiles = (a.s.G + kBNK - 1) / kBNK;
  const long long grid = (long long)a.s.B * a.s.Hkv * a.s.NG * a.tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  RopeTable rt{};
  if (ROPE) rt = *rope;
  hipLaunchKernelGGL((dkdv_kernel<D, ROPE>), dim3((unsigned)grid), dim3(kDkdvWaves * 64), 0, stream, a, rt);
  return hipGetLastError();
}

}  // namespace

#ifndef S2A_DQ_WAVES_LARGE
#define S2A_DQ_WAVES_LARGE 8  // waves per workgroup for groups longer than 2048
#endif

template <int D, bool ROPE>
hipError_t launch_dq_d(const BwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  if (a.s.G <= 2048) return launch_dq_t<D, 4, ROPE>(a, rope, stream);
  return launch_dq_t<D, S2A_DQ_WAVES_LARGE, ROPE>(a, rope, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  const bool r = rope != nullptr;
  if (a.s.D == 64) return r ? launch_dq_d<64, true>(a, rope, stream) : launch_dq_d<64, false>(a, rope, stream);
  return r ? launch_dq_d<128, true>(a, rope, stream) : launch_dq_d<128, false>(a, rope, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  const bool r = rope != nullptr;
  if (a.s.D == 64) return r ? launch_dkdv_t<64, true>(a, rope, stream) : launch_dkdv_t<64, false>(a, rope, stream);
  return r ? launch_dkdv_t<128, true>(a, rope, stream) : launch_dkdv_t<128, false>(a, rope, stream);
}

}  // namespace s2a
