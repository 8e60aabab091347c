// S2-Attn backward kernels for gfx950.
//
// The pages give no backward pass; this is the calculus of the forward
// definition (AIMech "LongLoRA and Shifted Sparse Attention (S^2-Attn)",
// opening definition), recomputing P from the saved log-sum-exp:
//   P = exp(S - lse),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - Delta),  dQ = c dS K,  dK = c dS^T Q,   c = 1/sqrt(D)
// per group of rolled rows.  Rows and keys are addressed at their original
// positions (the roll by -shift and its inverse folded into indices), so dQ,
// dK, dV land where the forward read q, k, v.
//
// Two kernels, no atomics (bitwise deterministic):
//   dkdv_kernel  one workgroup per (batch, k/v head, group, 128-key tile);
//                each wave owns 32 keys, keeps K and V as MFMA B operands in
//                VGPRs and accumulates dK^T, dV^T over every q head sharing
//                the k/v head and every 32-row q step from the diagonal to
//                the group end.  4 MFMA products per step.
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
    const float ang = (float)((r - floor(r)) * 6.283185307179586);
    float sn, cs;
    sincosf(ang, &sn, &cs);
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
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  using KStage = QuadStage<D, kBN, NT>;  // row-major (S^T) + transposed (dQ^T)
  using VStage = RowStage<D, kBN, NT>;   // row-major (dP^T)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * KStage::STR];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][D * KStage::TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kBN * VStage::STR];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const Shape& s = a.s;

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

  const int wave_q0 = t * BM + wave * 32;
  const int qi = wave_q0 + l32;
  const bool qvalid = qi < s.G;
  const int qpos = qvalid ? orig_pos(base, qi, s.N) : 0;
  const long long qoff = ((long long)(b * (long long)s.N + qpos) * s.H + h) * D;
  bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = as_bf16x8(qvalid ? ld16(a.q + qoff + kk * 16 + hh * 8) : zero_u4());
    dof[kk] = as_bf16x8(qvalid ? ld16(a.dout + qoff + kk * 16 + hh * 8) : zero_u4());
  }
  const long long stat_off = ((long long)b * s.H + h) * s.N + qpos;
  const float lse2 = qvalid ? a.lse[stat_off] * kLog2e : 0.f;
  const float dlt = qvalid ? a.delta[stat_off] : 0.f;

  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = zero16();

  const int rows_end = min((t + 1) * BM, s.G);
  const int ntiles = (rows_end + kBN - 1) / kBN;

  KStage kst;
  VStage vst;
  auto load_tile = [&](int n) {
    const int key0 = n * kBN;
    const uint16_t* kt = contig_tile(kb_ptr, kv_row, base, key0, kBN, s.G, s.N);
    if (kt != nullptr) {
      kst.load_contig(tid, kt, (int)kv_row);
      vst.load_contig(tid, vb_ptr + (kt - kb_ptr), (int)kv_row);
    } else {
      kst.load(tid, [&](int row) -> const uint16_t* {
        const int j = key0 + row;
        return j < s.G ? kb_ptr + orig_pos(base, j, s.N) * kv_row : nullptr;
      });
      vst.load(tid, [&](int row) -> const uint16_t* {
        const int j = key0 + row;
        return j < s.G ? vb_ptr + orig_pos(base, j, s.N) * kv_row : nullptr;
      });
    }
  };
  auto store_tile = [&](int buf) {
    kst.store(tid, Ks[buf], Kt[buf]);
    vst.store(tid, Vs[buf]);
  };

  auto compute = [&](int n, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int cur = n & 1;
    const int key0 = n * kBN;
    // S^T = K Q^T and dP^T = V dO^T: four independent accumulator chains,
    // interleaved; K and V fragments read from LDS one k-step ahead.
    f32x16 sc[kBN / 32], dp[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      sc[kb] = zero16();
      dp[kb] = zero16();
    }
    {
      const uint16_t* kp = &Ks[cur][l32 * KStage::STR + hh * 8];
      const uint16_t* vp = &Vs[cur][l32 * VStage::STR + hh * 8];
      bf16x8 kf[2][kBN / 32], vf[2][kBN / 32];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        kf[0][kb] = lds_frag(kp + kb * 32 * KStage::STR);
        vf[0][kb] = lds_frag(vp + kb * 32 * VStage::STR);
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + 1 < D / 16) {
#pragma unroll
          for (int kb = 0; kb < kBN / 32; ++kb) {
            kf[(kk + 1) & 1][kb] = lds_frag(kp + kb * 32 * KStage::STR + (kk + 1) * 16);
            vf[(kk + 1) & 1][kb] = lds_frag(vp + kb * 32 * VStage::STR + (kk + 1) * 16);
          }
        }
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb) {
          sc[kb] = mfma32x32x16(kf[kk & 1][kb], qf[kk], sc[kb]);
          dp[kb] = mfma32x32x16(vf[kk & 1][kb], dof[kk], dp[kb]);
        }
      }
    }
    bf16x8 dsb[kBN / 32][2];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(sc[kb][r] * a.scale_log2 - lse2);
        if constexpr (MASK) {
          const int j = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (j > qi) p = 0.f;
        }
        ds[r] = p * (dp[kb][r] - dlt);
      }
      dsb[kb][0] = cvt8(f32x8{ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]});
      dsb[kb][1] = cvt8(f32x8{ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]});
    }
    // dQ^T += K^T dS^T: D/32 independent output blocks cycled innermost.
    {
      const uint16_t* tp = &Kt[cur][l32 * KStage::TSTR + hh * 8];
      constexpr int KS = kBN / 16;
      bf16x8 tf[2][D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) tf[0][db] = lds_frag(tp + db * 32 * KStage::TSTR);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            tf[(ks + 1) & 1][db] = lds_frag(tp + db * 32 * KStage::TSTR + (ks + 1) * 16);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dq[db] = mfma32x32x16(tf[ks & 1][db], dsb[ks >> 1][ks & 1], dq[db]);
      }
    }
  };

  auto step = [&](int n, auto mask_tag) {
    if (n + 1 < ntiles) load_tile(n + 1);
    compute(n, mask_tag);
    if (n + 1 < ntiles) store_tile((n & 1) ^ 1);
    __syncthreads();
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // Unmasked tiles first, then the diagonal ones (see the forward kernel).
  const int n_full = min(ntiles, (wave_q0 + 1) / kBN);
  for (int n = 0; n < n_full; ++n) step(n, std::false_type{});
  for (int n = n_full; n < ntiles; ++n) step(n, std::true_type{});

  if (qvalid) store_row_acc<D, ROPE>(a.dq + qoff, dq, a.scale, hh, qpos, rope);
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int kDkdvWaves = 4;
constexpr int kBNK = kDkdvWaves * 32;  // keys per workgroup
constexpr int kBMQ = 32;               // q rows per step

template <int D, bool ROPE>
__global__ __launch_bounds__(kDkdvWaves * 64) void dkdv_kernel(BwdArgs a, RopeTable rope) {
  constexpr int NT = kDkdvWaves * 64;
  // Threads [0, NT/2) stage the q rows of a step, [NT/2, NT) the dout rows.
  using Stage = QuadStage<D, kBMQ, NT / 2>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][kBMQ * Stage::STR];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][D * Stage::TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Os[2][kBMQ * Stage::STR];
  __shared__ __attribute__((aligned(16))) uint16_t Ot[2][D * Stage::TSTR];
  __shared__ __attribute__((aligned(16))) float Lse2[2][kBMQ];
  __shared__ __attribute__((aligned(16))) float Dlt[2][kBMQ];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
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
  const int sh = (h0 >= (s.H >> 1)) ? s.shift : 0;  // shared by all rq q heads
  const int base = g * s.G + sh;
  const long long kv_row = (long long)s.Hkv * D;
  const long long q_row = (long long)s.H * D;

  // This lane's key: K and V rows as MFMA B operands.
  const int key_start = tk * kBNK;
  const int kw0 = key_start + wave * 32;
  const int kj = kw0 + l32;
  const bool kvalid = kj < s.G;
  const int kpos = kvalid ? orig_pos(base, kj, s.N) : 0;
  const long long koff = ((long long)b * s.N + kpos) * kv_row + (long long)kvh * D;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kf[kk] = as_bf16x8(kvalid ? ld16(a.k + koff + kk * 16 + hh * 8) : zero_u4());
    vf[kk] = as_bf16x8(kvalid ? ld16(a.v + koff + kk * 16 + hh * 8) : zero_u4());
  }

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  // Steps: every q head sharing this k/v head x every 32-row block from the
  // first row that can see this tile's keys to the group end.
  const int steps_per_head = (s.G - key_start + kBMQ - 1) / kBMQ;
  const int nsteps = steps_per_head * rq;

  const bool stage_dout = tid >= NT / 2;
  const int stid = tid & (NT / 2 - 1);
  Stage st;
  float stat = 0.f;
  auto load_step = [&](int step) {
    const int hi = step / steps_per_head;
    const int i0 = key_start + (step - hi * steps_per_head) * kBMQ;
    const int h = h0 + hi;
    const uint16_t* src = (stage_dout ? a.dout : a.q) + (long long)b * s.N * q_row + (long long)h * D;
    const uint16_t* tile = contig_tile(src, q_row, base, i0, kBMQ, s.G, s.N);
    if (tile != nullptr) {
      st.load_contig(stid, tile, (int)q_row);
    } else {
      st.load(stid, [&](int row) -> const uint16_t* {
        const int i = i0 + row;
        return i < s.G ? src + orig_pos(base, i, s.N) * q_row : nullptr;
      });
    }
    if (tid < 2 * kBMQ) {
      const int i = i0 + (tid & (kBMQ - 1));
      const long long so = ((long long)b * s.H + h) * s.N;
      if (tid < kBMQ)
        stat = i < s.G ? a.lse[so + orig_pos(base, i, s.N)] * kLog2e : INFINITY;
      else
        stat = i < s.G ? a.delta[so + orig_pos(base, i, s.N)] : 0.f;
    }
  };
  auto store_step = [&](int buf) {
    if (stage_dout)
      st.store(stid, Os[buf], Ot[buf]);
    else
      st.store(stid, Qs[buf], Qt[buf]);
    if (tid < kBMQ)
      Lse2[buf][tid] = stat;
    else if (tid < 2 * kBMQ)
      Dlt[buf][tid - kBMQ] = stat;
  };

  auto compute = [&](int step, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int cur = step & 1;
    const int hi = step / steps_per_head;
    const int i0 = key_start + (step - hi * steps_per_head) * kBMQ;
    // S = Q K^T and dP = dO V^T: lane column = this lane's key, elements run
    // over the step's rows 8*(r/4) + 4*hh + r%4.  Two independent chains,
    // fragments read one k-step ahead.
    f32x16 sc = zero16(), dp = zero16();
    {
      const uint16_t* qp = &Qs[cur][l32 * Stage::STR + hh * 8];
      const uint16_t* op = &Os[cur][l32 * Stage::STR + hh * 8];
      bf16x8 qa[2], oa[2];
      qa[0] = lds_frag(qp);
      oa[0] = lds_frag(op);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + 1 < D / 16) {
          qa[(kk + 1) & 1] = lds_frag(qp + (kk + 1) * 16);
          oa[(kk + 1) & 1] = lds_frag(op + (kk + 1) * 16);
        }
        sc = mfma32x32x16(qa[kk & 1], kf[kk], sc);
        dp = mfma32x32x16(oa[kk & 1], vf[kk], dp);
      }
    }
    float p[16], ds[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int row0 = 8 * r4 + 4 * hh;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Lse2[cur][row0]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Dlt[cur][row0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r4 * 4 + e;
        float pv = fast_exp2(sc[r] * a.scale_log2 - l4[e]);
        if constexpr (MASK) {
          if (kj > i0 + row0 + e) pv = 0.f;
        }
        p[r] = pv;
        ds[r] = pv * (dp[r] - d4[e]);
      }
    }
    bf16x8 pb[2], dsb[2];
    pb[0] = cvt8(f32x8{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]});
    pb[1] = cvt8(f32x8{p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]});
    dsb[0] = cvt8(f32x8{ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]});
    dsb[1] = cvt8(f32x8{ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]});
    // dV^T += dO^T P and dK^T += Q^T dS: 2*D/32 independent accumulators.
    {
      const uint16_t* otp = &Ot[cur][l32 * Stage::TSTR + hh * 8];
      const uint16_t* qtp = &Qt[cur][l32 * Stage::TSTR + hh * 8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 ofr[D / 32], qfr[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          ofr[db] = lds_frag(otp + db * 32 * Stage::TSTR + hf * 16);
          qfr[db] = lds_frag(qtp + db * 32 * Stage::TSTR + hf * 16);
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = mfma32x32x16(ofr[db], pb[hf], dv[db]);
          dk[db] = mfma32x32x16(qfr[db], dsb[hf], dk[db]);
        }
      }
    }
  };

  auto do_step = [&](int step, bool active, auto mask_tag) {
    if (step + 1 < nsteps) load_step(step + 1);
    if (active) compute(step, mask_tag);
    if (step + 1 < nsteps) store_step((step & 1) ^ 1);
    __syncthreads();
  };

  if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();

  // Per q head: steps whose rows all precede this wave's keys are skipped,
  // steps crossing the diagonal are masked, the rest run unmasked.  The step
  // sequence (and so the barrier count) is the same for every wave.
  const int skip = min(steps_per_head, (kw0 - key_start) / kBMQ);   // rows < kw0 only
  const int diag_end = min(steps_per_head, (kw0 + 31 - key_start) / kBMQ + 1);
  for (int hi = 0; hi < rq; ++hi) {
    const int s0 = hi * steps_per_head;
    for (int j = 0; j < skip; ++j) do_step(s0 + j, false, std::false_type{});
    for (int j = skip; j < diag_end; ++j) do_step(s0 + j, true, std::true_type{});
    for (int j = diag_end; j < steps_per_head; ++j) do_step(s0 + j, true, std::false_type{});
  }

  if (kvalid) {
    store_row_acc<D, ROPE>(a.dk + koff, dk, a.scale, hh, kpos, rope);
    store_row_acc<D, false>(a.dv + koff, dv, 1.f, hh, kpos, rope);
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

hipError_t launch_bwd_dq(const BwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  const bool r = rope != nullptr;
  if (a.s.D == 64) return r ? launch_dq_t<64, 4, true>(a, rope, stream) : launch_dq_t<64, 4, false>(a, rope, stream);
  return r ? launch_dq_t<128, 4, true>(a, rope, stream) : launch_dq_t<128, 4, false>(a, rope, stream);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, const RopeTable* rope, hipStream_t stream) {
  const bool r = rope != nullptr;
  if (a.s.D == 64) return r ? launch_dkdv_t<64, true>(a, rope, stream) : launch_dkdv_t<64, false>(a, rope, stream);
  return r ? launch_dkdv_t<128, true>(a, rope, stream) : launch_dkdv_t<128, false>(a, rope, stream);
}

}  // namespace s2a
