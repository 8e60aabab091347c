// Kernel parameter blocks and the host-side launchers of the S2-Attn kernels.
// Included by the C-ABI layer (host only) and by the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s2a {

// Shape of one call.  A "unit" is one (batch, q head, group) triple: one
// head's causal attention inside one group of G rolled rows.
struct Shape {
  int B, N, H, Hkv, D, G, shift;
  int NG;       // groups per head, N / G
  int pattern;  // which heads are shifted: 0 the second half, 1 alternate k/v heads (see head_shift)
};

// Frequencies of the RoPE pairs in revolutions per position:
// rev[i] = base^(-2i/D) / (pos_scale * 2*pi), float64 (D <= 128).
struct RopeTable {
  double rev[64];
};

struct FwdArgs {
  const uint16_t* q;  // [B, N, H, D]   (unrotated when rope is on)
  const uint16_t* k;  // [B, N, Hkv, D] (already rotated when rope is on)
  const uint16_t* v;  // [B, N, Hkv, D]
  uint16_t* out;      // [B, N, H, D]
  float* lse;         // [B, H, N] or nullptr
  Shape s;
  int tiles;          // q tiles per unit
  float scale_log2;   // log2(e) / sqrt(D)
};

struct BwdArgs {
  const uint16_t* q;     // [B, N, H, D]: without RoPE the caller's q, which the kernels scale by
                         // c * log2(e) with one bf16 rounding as they load it; with RoPE the
                         // rotate pass's bf16(rotated q * c * log2(e)).  Either way the operand of
                         // the forward's logits.
  const uint16_t* k;     // [B, N, Hkv, D] (rotated copy when rope is on)
  const uint16_t* v;
  const uint16_t* dout;  // [B, N, H, D]
  const float* nlse2;    // [B, H, N]: -lse * log2(e)        (written by the preprocess pass)
  const float* ndelta;   // [B, H, N]: -sum_d dout * out      (written by the preprocess pass)
  uint16_t* dq;          // [B, N, H, D]
  uint16_t* dk;          // [B, N, Hkv, D]
  uint16_t* dv;
  Shape s;
  int tiles;             // tiles per unit (q tiles for dQ, k tiles for dK/dV)
  float scale_log2;      // log2(e) / sqrt(D)
  float scale;           // 1 / sqrt(D)
};

// Launchers: enqueue on `stream`, return the HIP status of the launch.
hipError_t launch_fwd(const FwdArgs& a, const RopeTable* rope, hipStream_t stream);
hipError_t launch_bwd_delta(const uint16_t* out, const uint16_t* dout, const float* lse, float* ndelta,
                            float* nlse2, const Shape& s, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, const RopeTable* rope, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, const RopeTable* rope, hipStream_t stream);
// Rotate rows*heads*D bf16 values of a [B, N, heads, D] tensor into dst,
// multiplying by `scale` after the rotation (one bf16 rounding).
hipError_t launch_rope_rotate(const uint16_t* src, uint16_t* dst, const Shape& s, int heads,
                              const RopeTable& rope, float scale, hipStream_t stream);

}  // namespace s2a
