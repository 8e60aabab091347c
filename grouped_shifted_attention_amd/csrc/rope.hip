// RoPE with linear position interpolation, applied once per element into a
// workspace copy ("LoRA for Long-Context Adaptation", sections "Why vanilla
// LoRA under-delivers on long context" and "Position interpolation: the
// prerequisite"): pair (x[2i], x[2i+1]) of the row at original position p is
// rotated counter-clockwise by (p / s) * base^(-2i/D).
//
// Operands that the attention kernels stream many times (k in the forward
// and dQ passes, q in the dK/dV pass) are rotated here once instead of once
// per reuse; operands read once per workgroup are rotated inside the
// attention kernels with the same device routine.  The backward's q copy is
// also multiplied by c log2(e) here, in the same fp32 operations and order as
// the forward applies to its q rows, so both passes see identical logits.
// Memory-bound: one 16-byte load and store per thread, coalesced along D.
#include "device_common.hpp"
#include "kernels.hpp"

namespace s2a {

namespace {

template <int D>
__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                   long long rows, int N, int heads, RopeTable rope,
                                                   float scale) {
  constexpr int CH = D / 8;
  const long long item = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = rows * heads * CH;
  if (item >= total) return;
  const int ch = (int)(item % CH);
  const long long row = item / CH / heads;  // b*N + n
  const int pos = (int)(row % N);
  float x[8];
  unpack8(ld16(src + item * 8), x);
  rope_rotate8(x, pos, rope.rev, ch * 8, false);
  if (scale != 1.f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= scale;
  }
  st16(dst + item * 8, pack8(x));
}

}  // namespace

hipError_t launch_rope_rotate(const uint16_t* src, uint16_t* dst, const Shape& s, int heads,
                              const RopeTable& rope, float scale, hipStream_t stream) {
  const long long rows = (long long)s.B * s.N;
  const long long total = rows * heads * (s.D / 8);
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (s.D == 64)
    hipLaunchKernelGGL(rope_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, rows, s.N, heads, rope,
                       scale);
  else
    hipLaunchKernelGGL(rope_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, rows, s.N, heads, rope,
                       scale);
  return hipGetLastError();
}

}  // namespace s2a
