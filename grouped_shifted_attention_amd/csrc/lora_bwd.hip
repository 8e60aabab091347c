// Backward of the LoRA-adapted q/k/v projections, on bf16 MFMA (gfx950).
//
// Forward (lora_qkv.hip): T = s x A (kept, bf16, [M, 3r]) and
// y_p = x W_p + T_p B_p.  With the frozen W, the gradients for the upstream
// gradients dy_p are (the calculus of that forward; the pages do not spell
// out a backward):
//   dT_s = s dy_p B_p^T                  [M, 3r]   (K1, the three targets in one launch)
//   dx   = sum_p dy_p W_p^T + dT_s A^T   [M, d_in] (K1, one launch)
//   dB_p = T_p^T dy_p                    stored as B_p^T: [width_p, r] (K2 + K3)
//   dA_p = x^T dT_s,p                    stored as A_p^T: [r, d_in]   (K2 + K3)
// Weights arrive one row per output column (W_p^T [width_p, d_in],
// A_p^T [r, d_in], B_p^T [width_p, r]).
//
// K1 multiplies token rows (contiguous along the reduction) by a weight
// stored reduction-major ([k][n], contiguous along the output column): the
// weight tile sits in LDS as [64 k][256 n] and becomes MFMA A operands
// through transposing reads (ds_read_b64_tr_b16), the token tile as
// [256 m][64 k] read row-wise, as in the forward GEMM.  K2 contracts over the
// tokens, where both operands are token-major: both tiles are [64 m][cols]
// and both operands use transposing reads; the token range is split across
// workgroups into fp32 partial sums, which K3 adds in a fixed order
// (deterministic) and rounds to bf16.
#include <algorithm>

#include "device_common.hpp"
#include "lora_kernels.hpp"
#include "staging.hpp"

namespace s2a {
namespace {

// Transposing read of an MFMA operand whose k index is the LDS tile row:
// lane l receives tile column (col0 + l%32), rows k0 + 8*(l/32) + 0..7 in
// order.  Within each 16-lane group, lane i points at row k0 + 8hh + i/4 and
// the 4 columns col0 + 16*(group%2) + 4*(i%4) (lo read; the hi read is 4
// rows down).  With a row stride of 64 mod 256 bytes, the 4 rows x 2 column
// halves a 32-lane half reads fall in distinct 32-byte bank groups.
struct TrLane {
  int off;  // element offset of the lane's lo piece for k0 = 0, col0 = 0
  __device__ __forceinline__ TrLane(int lane, int rs) {
    const int g = lane >> 4, i = lane & 15;
    off = (8 * (g >> 1) + (i >> 2)) * rs + 16 * (g & 1) + 4 * (i & 3);
  }
  __device__ __forceinline__ bf16x8 read(const uint16_t* tile, int rs, int k0, int col0) const {
    const uint16_t* p = tile + k0 * rs + col0 + off;
    const s16x4 lo = lds_read_tr(p);
    const s16x4 hi = lds_read_tr(p + 4 * rs);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// ---------------------------------------------------------------------------
// K1: out[m][n] = scale * sum_segments sum_k tok[m][k] * w[k][n]
// ---------------------------------------------------------------------------
constexpr int kBM = 256, kBK = 64;
constexpr int kTokStride = kBK + 8;     // token tile row stride (elements)
constexpr int kTokElems = kBM * kTokStride;
// Row tiles per band of the walk order: the dx product reduces over all
// three targets' widths, so its token and weight panels are three times the
// forward's; bands of 4 row tiles (against 8) cut the backward call by 2-4%.
constexpr int kBand = 4;

// Output tile width BN: 256 (wide outputs; each wave 128 columns x 64
// tokens) or 64 (rank-wide outputs; each wave 64 columns x 32 tokens).
// Weight tile row stride BN + 32 elements: 576 or 192 bytes, whose first
// four rows fall at distinct 64-byte offsets mod 256.
template <int BN>
struct K1Shape {
  static constexpr int WStride = BN + 32;
  static constexpr int WElems = kBK * WStride;
  static constexpr int NI = BN == 256 ? 4 : 2;  // 32-column tiles per wave
  static constexpr int NJ = BN == 256 ? 2 : 1;  // 32-token tiles per wave
  static constexpr int WO = BN / (32 * NI);     // waves along the columns
  static constexpr int WChunks = BN / 8;        // 16-byte chunks per weight row
  static constexpr int WPer = kBK * WChunks / 512;
};

__device__ __forceinline__ void tile_coords(int id, int mt, int nt, int& tm, int& tn) {
  const int band = id / (kBand * nt);
  const int rem = id - band * kBand * nt;
  const int rows = min(kBand, mt - band * kBand);
  tn = rem / rows;
  tm = band * kBand + (rem - tn * rows);
}

// Up to three products of the same output shape in one launch, the product
// picked by blockIdx.y: the three s dy_p B_p^T products each have only
// ceil(M / 256) output tiles (r columns), too few to fill the chip alone.
struct LoraBwdK1Batch {
  LoraBwdK1Args arg[3];
};

template <int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void lora_bwd_k1(LoraBwdK1Batch batch) {
  const LoraBwdK1Args& a = batch.arg[blockIdx.y];
  using Sh = K1Shape<BN>;
  constexpr int kBN = BN;
  constexpr int kWStride = Sh::WStride;
  __shared__ __attribute__((aligned(16))) uint16_t X0[kTokElems];
  __shared__ __attribute__((aligned(16))) uint16_t X1[kTokElems];
  __shared__ __attribute__((aligned(16))) uint16_t W0[Sh::WElems];
  __shared__ __attribute__((aligned(16))) uint16_t W1[Sh::WElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int mt = (a.M + kBM - 1) / kBM;
  const int nt = (a.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(xcd_logical_id(blockIdx.x, mt * nt), mt, nt, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;

  // Reduction tiles: segment s contributes ceil(len_s / 64) tiles.
  int ntiles[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) ntiles[s] = s < a.nseg ? (a.seg[s].len + kBK - 1) / kBK : 0;
  const int kt_total = ntiles[0] + ntiles[1] + ntiles[2] + ntiles[3];

  // Staging map.  Token tile: chunk tc = tid%8 of rows tid/8 + 64 i.  Weight
  // tile: chunk wc (8 columns) of k rows wrow + (512 / chunks per row) i.
  const int tc = tid & 7, trow = tid >> 3;
  const int wc = tid % Sh::WChunks, wrow = tid / Sh::WChunks;
  constexpr int kWRowStep = 512 / Sh::WChunks;
  const int ncol = min(n0 + wc * 8, a.N - 8);  // clamped column (never stored past N)
  u32x4 xr[4], wr[Sh::WPer];
  int mrow[4];  // the thread's token rows (clamped)
#pragma unroll
  for (int i = 0; i < 4; ++i) mrow[i] = min(m0 + trow + 64 * i, a.M - 1);
  auto gload = [&](int kt) {
    // Segment of tile kt (wave-uniform; selected field by field so the
    // parameter block stays in scalar registers).
    int t = kt, s = 0;
    if (t >= ntiles[0]) { t -= ntiles[0]; s = 1; }
    if (s == 1 && t >= ntiles[1]) { t -= ntiles[1]; s = 2; }
    if (s == 2 && t >= ntiles[2]) { t -= ntiles[2]; s = 3; }
    const LoraBwdSeg g = s == 0 ? a.seg[0] : (s == 1 ? a.seg[1] : (s == 2 ? a.seg[2] : a.seg[3]));
    const int k0 = t * kBK;
    if (k0 + kBK <= g.len && g.stack >= g.len) {
      // A whole tile of one weight: no bounds checks, one pointer.
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = ld16(g.tok + (long long)mrow[i] * g.ldt + k0 + tc * 8);
      const uint16_t* wb = g.w[0] + (long long)k0 * g.ldw + ncol;
#pragma unroll
      for (int i = 0; i < Sh::WPer; ++i) wr[i] = ld16(wb + (wrow + kWRowStep * i) * g.ldw);
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mrow[i];
      const int k = k0 + tc * 8;
      const bool ok = k < g.len;
      const u32x4 v = ld16(g.tok + (long long)m * g.ldt + (ok ? k : 0));
      xr[i] = ok ? v : zero_u4();
    }
#pragma unroll
    for (int i = 0; i < Sh::WPer; ++i) {
      const int k = k0 + wrow + kWRowStep * i;
      const bool ok = k < g.len;
      const int kk = ok ? k : 0;
      // Stacked weights: g.stack rows per pointer, so kk < 3 * g.stack (and
      // g.stack = len for a single weight); two compares, no division.
      const int p = (kk >= g.stack) + (kk >= 2 * g.stack);
      const uint16_t* wp = p == 0 ? g.w[0] : (p == 1 ? g.w[1] : g.w[2]);
      const u32x4 v = ld16(wp + (long long)(kk - p * g.stack) * g.ldw + ncol);
      wr[i] = ok ? v : zero_u4();
    }
  };
  auto swrite = [&](uint16_t* xs, uint16_t* ws) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(xs + (trow + 64 * i) * kTokStride + tc * 8) = xr[i];
#pragma unroll
    for (int i = 0; i < Sh::WPer; ++i)
      *reinterpret_cast<u32x4*>(ws + (wrow + kWRowStep * i) * kWStride + wc * 8) = wr[i];
  };

  // Wave tile: output columns wo*32*NI + 32 i (A operands, transposing
  // reads), tokens wt*32*NJ + 32 j (B operands, row reads).
  constexpr int NI = Sh::NI, NJ = Sh::NJ;
  const int wo = wave % Sh::WO, wt = wave / Sh::WO;
  const TrLane tr(lane, kWStride);
  const int b_off = (wt * 32 * NJ + (lane & 31)) * kTokStride + 8 * (lane >> 5);
  f32x16 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = zero16();
  auto compute = [&](const uint16_t* xs, const uint16_t* ws) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[NI], bfr[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i) af[i] = tr.read(ws, kWStride, kk * 16, wo * 32 * NI + 32 * i);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[j] = lds_frag(xs + b_off + j * 32 * kTokStride + kk * 16);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  gload(0);
  swrite(X0, W0);
  lds_barrier();
  int kt = 0;
  for (; kt + 2 <= kt_total; kt += 2) {
    gload(kt + 1);
    compute(X0, W0);
    swrite(X1, W1);
    lds_barrier();
    if (kt + 2 < kt_total) gload(kt + 2);
    compute(X1, W1);
    if (kt + 2 < kt_total) swrite(X0, W0);
    lds_barrier();
  }
  if (kt < kt_total) compute(X0, W0);

  // Epilogue: lane = token, 4 runs of 4 consecutive output columns per tile.
  const float sc = a.scale;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int m = m0 + wt * 32 * NJ + 32 * j + (lane & 31);
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wo * 32 * NI + 32 * i + 8 * g + 4 * (lane >> 5);
        if (n < a.N) {
          const f32x16& v = acc[i][j];
          st8(a.out + (long long)m * a.ldo + n,
              cvt4_bits(v[4 * g] * sc, v[4 * g + 1] * sc, v[4 * g + 2] * sc, v[4 * g + 3] * sc));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K2: part[split][j][i] = sum over the split's tokens m of A[m][i] * B[m][j]
// ---------------------------------------------------------------------------
constexpr int kK2I = 128, kK2J = 64, kK2K = 64;
constexpr int kK2AStride = kK2I + 32;  // 320 B = 64 mod 256
constexpr int kK2BStride = kK2J + 32;  // 192 B: rows at 0, 192, 128, 64 mod 256

__global__ __launch_bounds__(256) void lora_bwd_k2(LoraBwdK2Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kK2K * kK2AStride];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kK2K * kK2BStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ti = (a.I + kK2I - 1) / kK2I, tj = (a.J + kK2J - 1) / kK2J;
  int id = blockIdx.x;
  const int split = id / (ti * tj);
  id -= split * ti * tj;
  const int bj = id / ti, bi = id - bj * ti;
  const int i0 = bi * kK2I, j0 = bj * kK2J;
  const int mbeg = split * a.rows_per_split;
  const int mend = min(a.M, mbeg + a.rows_per_split);

  // Staging: A tile 64 rows x 16 chunks (4 per thread), B tile 64 rows x 8
  // chunks (2 per thread).  Rows past the split end are zero.
  const TrLane tra(lane, kK2AStride), trb(lane, kK2BStride);
  f32x16 acc[2];
  acc[0] = zero16();
  acc[1] = zero16();
  for (int m0 = mbeg; m0 < mend; m0 += kK2K) {
    u32x4 av[4], bv[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int item = tid + 256 * q;
      const int row = item >> 4, c = item & 15;
      const int m = m0 + row;
      const int col = min(i0 + c * 8, a.I - 8);
      const u32x4 v = ld16(a.A + (long long)min(m, a.M - 1) * a.lda + col);
      av[q] = m < mend ? v : zero_u4();
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int item = tid + 256 * q;
      const int row = item >> 3, c = item & 7;
      const int m = m0 + row;
      const int col = min(j0 + c * 8, a.J - 8);
      const u32x4 v = ld16(a.B + (long long)min(m, a.M - 1) * a.ldb + col);
      bv[q] = m < mend ? v : zero_u4();
    }
    __syncthreads();  // previous tile's reads are done
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int item = tid + 256 * q;
      *reinterpret_cast<u32x4*>(As + (item >> 4) * kK2AStride + (item & 15) * 8) = av[q];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int item = tid + 256 * q;
      *reinterpret_cast<u32x4*>(Bs + (item >> 3) * kK2BStride + (item & 7) * 8) = bv[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kK2K / 16; ++kk) {
      const bf16x8 af = tra.read(As, kK2AStride, kk * 16, wave * 32);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
        acc[jb] = mfma32x32x16(af, trb.read(Bs, kK2BStride, kk * 16, jb * 32), acc[jb]);
    }
  }

  // C[i][j]: lane -> j = 32 jb + lane%32, element r -> i = 32 wave + 8(r/4) + 4hh + r%4.
  const int hh = lane >> 5;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int j = j0 + jb * 32 + (lane & 31);
    if (j >= a.J) continue;
    float* dst = a.part + ((long long)split * a.J + j) * a.I;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int i = i0 + wave * 32 + 8 * g + 4 * hh;
      if (i < a.I)
        *reinterpret_cast<f32x4*>(dst + i) =
            f32x4{acc[jb][4 * g], acc[jb][4 * g + 1], acc[jb][4 * g + 2], acc[jb][4 * g + 3]};
    }
  }
}

// K3: out[i * si + j * sj] = bf16(sum_split part[split][j][i]), splits added
// in order.
__global__ __launch_bounds__(256) void lora_bwd_k3(const float* __restrict__ part, int splits, int I, int J,
                                                   uint16_t* __restrict__ out, long long si, long long sj) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)I * J) return;
  const int i = (int)(idx % I), j = (int)(idx / I);
  float sum = 0.f;
  for (int s = 0; s < splits; ++s) sum += part[((long long)s * J + j) * I + i];
  const u32x2 w = cvt4_bits(sum, 0.f, 0.f, 0.f);
  out[i * si + j * sj] = (uint16_t)(w[0] & 0xffffu);
}

// `count` products of the same M and N (batch.arg[0 .. count-1]).
template <int BN>
hipError_t launch_k1(const LoraBwdK1Batch& batch, int count, hipStream_t stream) {
  const LoraBwdK1Args& a = batch.arg[0];
  const long long grid = (long long)((a.M + kBM - 1) / kBM) * ((a.N + BN - 1) / BN);
  if (grid <= 0 || count <= 0) return hipSuccess;
  hipLaunchKernelGGL(lora_bwd_k1<BN>, dim3((unsigned)grid, (unsigned)count), dim3(512), 0, stream, batch);
  return hipGetLastError();
}

hipError_t launch_k2k3(const LoraBwdK2Args& a, uint16_t* out, long long si, long long sj, hipStream_t stream) {
  const long long tiles = (long long)((a.I + kK2I - 1) / kK2I) * ((a.J + kK2J - 1) / kK2J);
  const int splits = (a.M + a.rows_per_split - 1) / a.rows_per_split;
  if (tiles <= 0 || splits <= 0) return hipSuccess;
  hipLaunchKernelGGL(lora_bwd_k2, dim3((unsigned)(tiles * splits)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)a.I * a.J;
  hipLaunchKernelGGL(lora_bwd_k3, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.part, splits, a.I, a.J,
                     out, si, sj);
  return hipGetLastError();
}

}  // namespace

int lora_bwd_splits(int M) {
  // About 1024 tokens per split, at most 64 splits.
  return M <= 0 ? 0 : std::min(64, (M + 1023) / 1024);
}

hipError_t launch_lora_qkv_bwd(const LoraQkvBwdArgs& q, hipStream_t stream) {
  if (q.M == 0) return hipSuccess;
  hipError_t e;
  if (q.r > 0) {
    // dT_s = s dy_p B_p^T into the workspace, target p in columns p r ..
    // (the three products in one launch).
    LoraBwdK1Batch kb{};
    for (int p = 0; p < 3; ++p) {
      LoraBwdK1Args& k = kb.arg[p];
      k.M = q.M;
      k.N = q.r;
      k.out = q.dts + p * q.r;
      k.ldo = 3 * q.r;
      k.scale = q.scale;
      k.nseg = 1;
      k.seg[0] = LoraBwdSeg{q.dy[p], q.width[p], {q.bt[p], q.bt[p], q.bt[p]}, q.r, q.width[p], q.width[p]};
    }
    if ((e = launch_k1<64>(kb, 3, stream)) != hipSuccess) return e;
  }
  // dx = sum_p dy_p W_p^T (+ dT_s A^T).
  LoraBwdK1Batch xb{};
  LoraBwdK1Args& k = xb.arg[0];
  k.M = q.M;
  k.N = q.K;
  k.out = q.dx;
  k.ldo = q.K;
  k.scale = 1.f;
  k.nseg = 0;
  for (int p = 0; p < 3; ++p)
    k.seg[k.nseg++] = LoraBwdSeg{q.dy[p], q.width[p], {q.wt[p], q.wt[p], q.wt[p]}, q.K, q.width[p], q.width[p]};
  if (q.r > 0) k.seg[k.nseg++] = LoraBwdSeg{q.dts, 3 * q.r, {q.at[0], q.at[1], q.at[2]}, q.K, 3 * q.r, q.r};
  if ((e = launch_k1<256>(xb, 1, stream)) != hipSuccess) return e;
  if (q.r == 0) return hipSuccess;
  const int splits = lora_bwd_splits(q.M);
  const int rps = ((q.M + splits - 1) / splits + kK2K - 1) / kK2K * kK2K;
  for (int p = 0; p < 3; ++p) {
    // dB_p^T[o][j] = sum_m dy_p[m][o] T[m][p r + j]  (I = width_p, J = r)
    LoraBwdK2Args b{q.dy[p], q.width[p], q.t + p * q.r, 3 * q.r, q.M, q.width[p], q.r, rps, q.part};
    if ((e = launch_k2k3(b, q.dbt[p], q.r, 1, stream)) != hipSuccess) return e;
    // dA_p^T[j][n] = sum_m dT_s[m][p r + j] x[m][n]  (I = d_in, J = r)
    LoraBwdK2Args c{q.x, q.K, q.dts + p * q.r, 3 * q.r, q.M, q.K, q.r, rps, q.part};
    if ((e = launch_k2k3(c, q.dat[p], 1, q.K, stream)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace s2a
