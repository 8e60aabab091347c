// Device helpers shared by the S2-Attn kernels for gfx950 (CDNA4).
//
// Matrix products use v_mfma_f32_32x32x16_bf16.  For that instruction a
// wave64 holds
//   A (32 x 16):  lane l -> row l%32, k = 8*(l/32) + s for element s = 0..7
//   B (16 x 32):  lane l -> col l%32, k = 8*(l/32) + s
//   C (32 x 32):  lane l -> col l%32, element r = 0..15 -> row 8*(r/4) + 4*(l/32) + r%4
// A product whose reduction index is permuted identically in A and B is
// unchanged, which the kernels use to feed a C tile straight back in as a
// B operand without moving data between lanes (the matching A operand is
// read with ds_read_b64_tr_b16 in that permuted row order).
#pragma once

#include "kernels.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s2a {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, WGs dispatched round-robin
constexpr int kCusPerXcd = 32;  // MI355X: 256 compute units over the 8 dies

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 16-byte global load / store of 8 bf16 (as raw bits).
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(uint16_t* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round 8 floats to bf16 (round-to-nearest-even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 cvt8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
// The part of x that its bf16 rounding hi misses, itself rounded to bf16:
// hi + lo carries x to about 16 significant bits, so a product taken as
// A*hi + A*lo on bf16 MFMA is as accurate as one with an fp32 operand.
__device__ __forceinline__ bf16x8 bf16_residual8(f32x8 x, bf16x8 hi) {
  return cvt8(x - __builtin_convertvector(hi, f32x8));
}
__device__ __forceinline__ u32x2 cvt4_bits(float a, float b, float c, float d) {
  f32x4 x = {a, b, c, d};
  return __builtin_bit_cast(u32x2, __builtin_convertvector(x, bf16x4));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Reductions across the two wave halves (lanes l and l^32), which hold the
// two halves of one row of a C tile.  v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second; with both
// operands equal to x, every lane ends up with {x[l], x[l^32]} spread over
// the two results, so combining the two results is the pair reduction.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are dispatched round-robin over the XCDs (blockIdx % 8).  Map
// the hardware id to a logical id so that each XCD receives one contiguous
// range of logical work items: tiles of one attention unit then share that
// XCD's L2.  A bijection on [0, total).
__device__ __forceinline__ int xcd_logical_id(int id, int total) {
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = id % kXcds, local = id / kXcds;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Shift of q head h.  Pattern 0: the second half of the heads (h >= H/2)
// is shifted ("LongLoRA and Shifted Sparse Attention (S^2-Attn)", opening
// definition).  Pattern 1: alternate heads ("LoRA for Long-Context
// Adaptation", section "Shifted sparse attention"), read as the q heads of
// the odd k/v heads, which is the odd heads without sharing and keeps every
// k/v head's rows rolled one way.
__device__ __forceinline__ int head_shift(int h, const Shape& s) {
  const bool shifted = s.pattern ? ((h / (s.H / s.Hkv)) & 1) != 0 : h >= (s.H >> 1);
  return shifted ? s.shift : 0;
}

// Unit (b, q head h, group g) of a forward or dQ workgroup, from the unit
// index.  The q heads that share a k/v head are adjacent (order b, k/v head,
// g, q head within the k/v head), so consecutive units -- one XCD's
// contiguous range of work items -- read the same k/v rows and share them in
// L2.  Without grouped-query sharing this is the order (b, h, g).
struct QUnit {
  int b, h, g;
};
__device__ __forceinline__ QUnit decode_q_unit(int unit, const Shape& s) {
  const int rq = s.H / s.Hkv;
  const int hi = unit % rq, rest = unit / rq;
  const int g = rest % s.NG, bk = rest / s.NG;
  return QUnit{bk / s.Hkv, (bk % s.Hkv) * rq + hi, g};
}

// Original sequence position of local row j of a group whose first rolled
// row sits at `base` = g*G + shift_h (< N).  The roll by -shift is circular
// and base + j < 2N, so one conditional subtraction folds it.
__device__ __forceinline__ int orig_pos(int base, int j, int N) {
  const int p = base + j;
  return p >= N ? p - N : p;
}

// Sine and cosine of an angle given in turns, t in [0, 1]: the hardware's
// v_sin_f32 / v_cos_f32 take their argument in turns.
__device__ __forceinline__ void sincos_turns(float t, float& sn, float& cs) {
  sn = __builtin_amdgcn_sinf(t);
  cs = __builtin_amdgcn_cosf(t);
}

// RoPE: rotate the 4 pairs held in 8 consecutive bf16 (d0 .. d0+7, d0 even)
// of a row at original position `pos`.  rev[i] = base^(-2i/D) / (s * 2*pi)
// is the pair's frequency in revolutions per position; the angle is reduced
// to a fraction of a turn in float64 before the float32 sine and cosine.
__device__ __forceinline__ void rope_rotate8(float x[8], int pos, const double* rev, int d0, bool inverse) {
  const double p = (double)pos;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double r = p * rev[(d0 >> 1) + e];
    float sn, cs;
    sincos_turns((float)(r - floor(r)), sn, cs);
    if (inverse) sn = -sn;
    const float a = x[2 * e], b = x[2 * e + 1];
    x[2 * e] = a * cs - b * sn;
    x[2 * e + 1] = a * sn + b * cs;
  }
}

__device__ __forceinline__ void unpack8(u32x4 v, float x[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    x[2 * w] = bf16lo(v[w]);
    x[2 * w + 1] = bf16hi(v[w]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float x[8]) {
  f32x8 f = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_bit_cast(u32x4, cvt8(f));
}

// 8 bf16 values times a scale, rounded back to bf16 once.
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float scale) {
  float x[8];
  unpack8(v, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= scale;
  return pack8(x);
}

}  // namespace s2a
