// LoRA-adapted q/k/v projections ahead of S2-Attn, on bf16 MFMA (gfx950).
//
// For each target p in (q, k, v), with token rows x [M, K]:
//   y_p = x W_p + s (x A_p) B_p
// ("LoRA for Long-Context Adaptation", section "Why vanilla LoRA
// under-delivers on long context": the frozen projection plus the product of
// the two small trained matrices, read with token rows as row vectors; the
// pages name no scale, s is the caller's).  Weights arrive one row per output
// column (W_p^T [width_p, K], A_p^T [r, K], B_p^T [width_p, r]), so every
// operand of every product is contiguous along its reduction index.
//
// Two launches of one GEMM kernel:
//   1. T = s x [A_q A_k A_v]  -> [M, 3r] bf16 (the three adapters' rows
//      stacked into one 3r-row weight);
//   2. y_p = x W_p + T_p B_p, the low-rank term as ceil(r/64) extra
//      reduction tiles after the K/64 tiles of the frozen weight, so the
//      update costs no extra pass over y.
//
// The kernel computes Y^T tiles: MFMA A operand = weight rows (32 output
// columns), B operand = token rows (32 tokens), so an accumulator lane holds
// one token and runs of 4 consecutive output columns, stored as 8-byte runs
// into the row-major [M, width] outputs (= [B, N, heads, D] rows).
//
// Tiling: 256 tokens x 256 output columns per workgroup, K in tiles of 64.
// 8 waves (2 per SIMD), each 64 tokens x 128 columns = 2 x 4 MFMA tiles of
// 32 x 32, reading 6 operand fragments per 16-deep step for 8 MFMAs.  Tiles
// are staged global -> VGPR -> LDS, double buffered (one tile in flight
// while the other is multiplied), rows padded to 72 elements so 16
// consecutive rows start in 16 distinct 4-bank groups (conflict-free 16-byte
// operand reads).  Workgroups walk the output in bands of 8 row tiles,
// column-major inside a band, and each XCD takes one contiguous range of that
// order, so the 32 workgroups an XCD runs at once share 8 token panels and 4
// weight panels in its L2.
#include "device_common.hpp"
#include "lora_kernels.hpp"
#include "staging.hpp"

namespace s2a {
namespace {

constexpr int kBM = 256;   // tokens per workgroup tile
constexpr int kBN = 256;   // output columns per workgroup tile
constexpr int kBK = 64;    // reduction depth per staged tile
constexpr int kLdsStride = kBK + 8;
constexpr int kTileElems = kBM * kLdsStride;  // one operand tile in LDS
constexpr int kBand = 8;   // row tiles per band of the walk order

// Logical tile id -> (row tile, column tile): bands of kBand row tiles,
// column-major inside a band.
__device__ __forceinline__ void tile_coords(int id, int mt, int nt, int& tm, int& tn) {
  const int band = id / (kBand * nt);
  const int rem = id - band * kBand * nt;
  const int rows = min(kBand, mt - band * kBand);
  tn = rem / rows;
  tm = band * kBand + (rem - tn * rows);
}

// STACKED: the weight rows of the single segment are the rows of w[0], w[1],
// w[2] stacked, `stack` rows each (the adapters' A^T for the T product).
template <bool STACKED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void lora_gemm_kernel(LoraGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs0[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t Xs1[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t Ws0[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t Ws1[kTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int mt = (a.M + kBM - 1) / kBM;
  const int nt = a.tile_start[3];
  int tm, tn;
  tile_coords(xcd_logical_id(blockIdx.x, mt * nt), mt, nt, tm, tn);
  const int seg = tn >= a.tile_start[2] ? 2 : (tn >= a.tile_start[1] ? 1 : 0);
  const int m0 = tm * kBM;
  const int n0 = (tn - a.tile_start[seg]) * kBN;  // first output column inside the segment
  const int width = a.width[seg];
  const int K = a.K;
  const int kx = K / kBK;                              // tiles of the frozen weight

  // Staging map: thread -> chunk c (8 elements) of rows srow + 64*i.
  const int c = tid & 7, srow = tid >> 3;
  int xoff[4];            // element offsets of the thread's x rows (clamped to M-1)
  int trow[4];            // token rows (for the LoRA tail), clamped
  int wrow[4];            // weight rows inside the segment, clamped
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = min(m0 + srow + 64 * i, a.M - 1);
    trow[i] = m;
    xoff[i] = (m - m0) * K + c * 8;
    wrow[i] = min(n0 + srow + 64 * i, width - 1);
  }
  const uint16_t* xbase = a.x + (long long)m0 * K;
  const uint16_t* wseg = a.w[seg];
  const uint16_t* wbase = wseg + (long long)n0 * K;
  int woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) woff[i] = (wrow[i] - n0) * K + c * 8;

  // Stacked mode: row pointers into the three adapters.
  const uint16_t* wptr[4];
  if constexpr (STACKED) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = wrow[i] / a.stack;
      wptr[i] = a.w[p] + (long long)(wrow[i] - p * a.stack) * K + c * 8;
    }
  }

  u32x4 xr[4], wr[4];
  auto gload = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = ld16(xbase + xoff[i] + k0);
    if constexpr (STACKED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[i] = ld16(wptr[i] + k0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[i] = ld16(wbase + woff[i] + k0);
    }
  };
  // LoRA tail tile u: token rows of T (this segment's r columns) against
  // B_p^T.  Chunks past the rank load an in-bounds chunk and are zeroed.
  auto gload_tail = [&](int u) {
    const int j = u * kBK + c * 8;  // adapter index of the chunk
    const bool ok = j < a.r;
    const int jj = ok ? j : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 tv = ld16(a.t + (long long)trow[i] * a.ldt + seg * a.r + jj);
      const u32x4 bv = ld16(a.bt[seg] + (long long)wrow[i] * a.r + jj);
      xr[i] = ok ? tv : zero_u4();
      wr[i] = ok ? bv : zero_u4();
    }
  };
  auto swrite = [&](uint16_t* xs, uint16_t* ws) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(xs + (srow + 64 * i) * kLdsStride + c * 8) = xr[i];
      *reinterpret_cast<u32x4*>(ws + (srow + 64 * i) * kLdsStride + c * 8) = wr[i];
    }
  };

  // Wave tile: output columns wo*128 + 32*i (i < 4), tokens wt*64 + 32*j (j < 2).
  const int wo = wave & 1, wt = wave >> 1;
  const int a_off = (wo * 128 + (lane & 31)) * kLdsStride + 8 * (lane >> 5);
  const int b_off = (wt * 64 + (lane & 31)) * kLdsStride + 8 * (lane >> 5);
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

  auto compute = [&](const uint16_t* xs, const uint16_t* ws) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = lds_frag(ws + a_off + i * 32 * kLdsStride + kk * 16);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = lds_frag(xs + b_off + j * 32 * kLdsStride + kk * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
      // Keep each step's operand reads next to its products (hoisting all of
      // them costs 72 VGPRs the accumulators need).
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  gload(0);
  swrite(Xs0, Ws0);
  lds_barrier();
  int kt = 0;
  for (; kt + 2 <= kx; kt += 2) {
    gload(kt + 1);
    compute(Xs0, Ws0);
    swrite(Xs1, Ws1);
    lds_barrier();
    if (kt + 2 < kx) gload(kt + 2);
    compute(Xs1, Ws1);
    if (kt + 2 < kx) swrite(Xs0, Ws0);
    lds_barrier();
  }
  if (kt < kx) {  // odd K/64: the last tile sits in buffer 0
    compute(Xs0, Ws0);
    lds_barrier();
  }
  if constexpr (!STACKED) {
    // The low-rank term: ceil(r/64) more reduction tiles, unpipelined (one or
    // two tiles against K/64).  The last barrier above freed both buffers.
    for (int u = 0; u * kBK < a.r; ++u) {
      gload_tail(u);
      swrite(Xs0, Ws0);
      lds_barrier();
      compute(Xs0, Ws0);
      lds_barrier();
    }
  }

  // Epilogue: lane = token, 4 runs of 4 consecutive output columns per tile.
  uint16_t* y = a.y[seg];
  const int ldy = a.ldy[seg];
  const float sc = a.scale;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wt * 64 + 32 * j + (lane & 31);
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int o = n0 + wo * 128 + 32 * i + 8 * g + 4 * (lane >> 5);
        if (o < width) {
          const f32x16& v = acc[i][j];
          st8(y + (long long)m * ldy + o,
              cvt4_bits(v[4 * g] * sc, v[4 * g + 1] * sc, v[4 * g + 2] * sc, v[4 * g + 3] * sc));
        }
      }
    }
  }
}

template <bool STACKED>
hipError_t launch_gemm(const LoraGemmArgs& a, hipStream_t stream) {
  const long long mt = (a.M + kBM - 1) / kBM;
  const long long grid = mt * a.tile_start[3];
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(lora_gemm_kernel<STACKED>, dim3((unsigned)grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int lora_col_tiles(int width) { return (width + kBN - 1) / kBN; }

hipError_t launch_lora_qkv(const LoraQkvArgs& q, hipStream_t stream) {
  if (q.M == 0) return hipSuccess;
  if (q.r > 0) {
    // T = s x [A_q A_k A_v]: one segment of 3r weight rows.
    LoraGemmArgs t{};
    t.x = q.x;
    t.M = q.M;
    t.K = q.K;
    for (int p = 0; p < 3; ++p) t.w[p] = q.at[p];
    t.stack = q.r;
    t.width[0] = 3 * q.r;
    t.y[0] = q.t;
    t.ldy[0] = 3 * q.r;
    t.tile_start[0] = 0;
    t.tile_start[1] = t.tile_start[2] = t.tile_start[3] = lora_col_tiles(3 * q.r);
    t.scale = q.scale;
    hipError_t e = launch_gemm<true>(t, stream);
    if (e != hipSuccess) return e;
  }
  LoraGemmArgs g{};
  g.x = q.x;
  g.M = q.M;
  g.K = q.K;
  g.tile_start[0] = 0;
  for (int p = 0; p < 3; ++p) {
    g.w[p] = q.wt[p];
    g.width[p] = q.width[p];
    g.y[p] = q.y[p];
    g.ldy[p] = q.width[p];
    g.bt[p] = q.bt[p];
    g.tile_start[p + 1] = g.tile_start[p] + lora_col_tiles(q.width[p]);
  }
  g.t = q.t;
  g.ldt = 3 * q.r;
  g.r = q.r;
  g.scale = 1.f;
  return launch_gemm<false>(g, stream);
}

}  // namespace s2a
