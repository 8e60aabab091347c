// Backward pre-pass: the row statistics the dK/dV and dQ kernels start their
// MFMA accumulators from,
//   ndelta[b, h, n] = -sum_d dout[b, n, h, d] * out[b, n, h, d]
//   nlse2[b, h, n]  = -lse[b, h, n] * log2(e).
// The softmax backward needs, per row i, Delta_i = sum_j P_ij dP_ij, which
// equals dO_i . O_i because O_i = sum_j P_ij V_j and dP_ij = dO_i . V_j.
// Computing it once per row here spares the dK/dV pass (which visits every
// row once per k/v tile) from re-reading O.  Storing both statistics negated
// (and lse in log2 units) lets the later kernels use them as the start value
// of the S and dP accumulators: P = exp2(acc), dS = P * acc.
// HBM-bound: reads out and dout once with 16-byte coalesced loads, and 8
// bytes per row else.
#include "device_common.hpp"
#include "kernels.hpp"

namespace s2a {

namespace {

// One row (one (b, n, h)) per group of D/8 lanes; each lane dots 8 elements.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ out, const uint16_t* __restrict__ dout,
                                                    const float* __restrict__ lse, float* __restrict__ ndelta,
                                                    float* __restrict__ nlse2, long long rows, int N, int H) {
  constexpr int CH = D / 8;  // lanes per row (16 or 8), a power of two dividing 64
  const long long item = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = item / CH;  // (b*N + n)*H + h
  float acc = 0.f;
  if (row < rows) {
    float x[8], y[8];
    unpack8(ld16(out + item * 8), x);
    unpack8(ld16(dout + item * 8), y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += x[e] * y[e];
  }
#pragma unroll
  for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && (item % CH) == 0) {
    const int h = (int)(row % H);
    const long long bn = row / H;
    const long long b = bn / N;
    const int n = (int)(bn % N);
    const long long o = (b * H + h) * N + n;
    ndelta[o] = -acc;
    nlse2[o] = -lse[o] * kLog2e;
  }
}

}  // namespace

hipError_t launch_bwd_delta(const uint16_t* out, const uint16_t* dout, const float* lse, float* ndelta,
                            float* nlse2, const Shape& s, hipStream_t stream) {
  const long long rows = (long long)s.B * s.N * s.H;
  const long long total = rows * (s.D / 8);
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (s.D == 64)
    hipLaunchKernelGGL(delta_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, out, dout, lse, ndelta, nlse2,
                       rows, s.N, s.H);
  else
    hipLaunchKernelGGL(delta_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, out, dout, lse, ndelta, nlse2,
                       rows, s.N, s.H);
  return hipGetLastError();
}

}  // namespace s2a
