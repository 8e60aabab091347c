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

int lora_col_tiles(int width);
hipError_t launch_lora_qkv(const LoraQkvArgs& a, hipStream_t stream);

}  // namespace s2a
