// Parameter blocks and launcher of the LoRA q/k/v projection kernels.
// Included by the C-ABI layer (host only) and by the kernel source.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s2a {

// One call of the projection: y_p = x W_p + s (x A_p) B_p for p = q, k, v.
struct LoraQkvArgs {
  const uint16_t* x;      // [M, K] token rows
  int M, K;               // K a multiple of 64
  const uint16_t* wt[3];  // W_p^T [width_p, K]
  const uint16_t* at[3];  // A_p^T [r, K]       (unused when r == 0)
  const uint16_t* bt[3];  // B_p^T [width_p, r] (unused when r == 0)
  int width[3];           // output columns per target, multiples of 64
  int r;                  // adapter rank, a multiple of 8, or 0
  float scale;            // s
  uint16_t* y[3];         // [M, width_p]
  uint16_t* t;            // [M, 3r] workspace: s x A_p for the three targets side by side
};

// One GEMM launch: Y = scale * (x W^T [+ T B^T]) over up to three column
// segments (one per target), each with its own weight, output and adapter.
struct LoraGemmArgs {
  const uint16_t* x;
  int M, K;
  const uint16_t* w[3];   // segment weights [width, K] (stacked mode: the three A^T, `stack` rows each)
  int width[3];
  uint16_t* y[3];
  int ldy[3];
  int tile_start[4];      // prefix sums of the segments' column tiles
  const uint16_t* t;      // LoRA tail operand [M, ldt]; segment p uses columns p*r .. p*r+r-1
  int ldt;
  int r;                  // 0: no tail
  const uint16_t* bt[3];  // [width, r]
  int stack;
  float scale;
};

// Backward.  A reduction segment of the token-by-weight product: token rows
// tok[m][k] (row stride ldt) against weight rows w[k][n] (row stride ldw),
// k < len; the weight rows come from w[0], w[1], w[2] in turn, `stack` rows
// each (stack = len for a single weight).
struct LoraBwdSeg {
  const uint16_t* tok;
  int ldt;
  const uint16_t* w[3];
  int ldw;
  int len;
  int stack;
};

// out[m][n] = scale * sum over segments of tok . w, m < M, n < N.
struct LoraBwdK1Args {
  int M, N;
  uint16_t* out;
  int ldo;
  float scale;
  int nseg;
  LoraBwdSeg seg[4];
};

// part[split][j][i] = sum over the split's rows m of A[m][i] * B[m][j].
struct LoraBwdK2Args {
  const uint16_t* A;
  int lda;
  const uint16_t* B;
  int ldb;
  int M, I, J;
  int rows_per_split;
  float* part;
};

struct LoraQkvBwdArgs {
  const uint16_t* x;      // [M, K]
  int M, K;
  const uint16_t* wt[3];  // W_p^T [width_p, K]
  const uint16_t* at[3];  // A_p^T [r, K]
  const uint16_t* bt[3];  // B_p^T [width_p, r]
  int width[3];
  int r;
  float scale;
  const uint16_t* t;      // the forward's s x A, [M, 3r]
  const uint16_t* dy[3];  // upstream gradients [M, width_p]
  uint16_t* dx;           // [M, K]
  uint16_t* dat[3];       // dA_p^T [r, K]
  uint16_t* dbt[3];       // dB_p^T [width_p, r]
  uint16_t* dts;          // workspace [M, 3r]: s dy_p B_p^T
  float* part;            // workspace: split partial sums
};

int lora_col_tiles(int width);
int lora_bwd_splits(int M);
hipError_t launch_lora_qkv_bwd(const LoraQkvBwdArgs& a, hipStream_t stream);
hipError_t launch_lora_qkv(const LoraQkvArgs& a, hipStream_t stream);

}  // namespace s2a
