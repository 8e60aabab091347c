"""Seeded synthetic inputs and the workload shapes for S2-Attn.

This module is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the attention method itself: it only
draws random numbers, rounds them to bfloat16 and widens bfloat16 back to
float64, so both sides of every parity check see bit-identical inputs.

Input recipe: ``numpy.random.default_rng(seed)`` (PCG64), draws in the order
q, k, v, dout, each ``standard_normal(shape, float32)``, rounded to bfloat16
with round-to-nearest-even.  q/dout are [B, N, H, D] and k/v are
[B, N, Hkv, D], contiguous.  These stand in for projected LLaMA2 attention
activations on long documents; no dataset or trained weight is used.
"""
from __future__ import annotations

import numpy as np

# Workload shapes.  Sizes are the LLaMA2-7B and 70B attention shapes the pages
# fine-tune at (LongLoRA abstract: 7B to 100k, 70B to 32k), always with the
# group size G = N/4 that the AIMech page's group-size limitation recommends
# and the shift G/2 of the AIMech definition.
WORKLOADS = {
    "tiny_n256": dict(B=1, N=256, H=4, Hkv=4, D=64, G=64, shift=32, rope=None),
    "llama2_7b_n8k": dict(B=1, N=8192, H=32, Hkv=32, D=128, G=2048, shift=1024, rope=None),
    "llama2_7b_n32k": dict(B=1, N=32768, H=32, Hkv=32, D=128, G=8192, shift=4096, rope=None),
    "llama2_7b_n100k": dict(B=1, N=102400, H=32, Hkv=32, D=128, G=25600, shift=12800, rope=None),
    "llama2_70b_gqa_n32k_rope": dict(B=1, N=32768, H=64, Hkv=8, D=128, G=8192, shift=4096,
                                     rope=(10000.0, 8.0)),
    # Dense causal attention (one group, no shift): the inference mode the
    # pages switch back to after S2-Attn fine-tuning.
    "llama2_7b_dense_n32k": dict(B=1, N=32768, H=32, Hkv=32, D=128, G=32768, shift=0, rope=None),
    # 100k context with position interpolation by s = 25 (a 4k model
    # stretched to 100k), and 32k with the RoPE base scaled by 8 instead.
    "llama2_7b_n100k_rope_pi25": dict(B=1, N=102400, H=32, Hkv=32, D=128, G=25600, shift=12800,
                                      rope=(10000.0, 25.0)),
    "llama2_7b_n32k_rope_base8": dict(B=1, N=32768, H=32, Hkv=32, D=128, G=8192, shift=4096,
                                      rope=(80000.0, 1.0)),
    # Alternate heads shifted instead of the second half (the variant of the
    # "LoRA for Long-Context Adaptation" page).
    "llama2_7b_n32k_alternate": dict(B=1, N=32768, H=32, Hkv=32, D=128, G=8192, shift=4096, rope=None,
                                     head_pattern="alternate"),
}

# The workload the benchmark times: LLaMA2-7B attention at 32k context.
BENCH_WORKLOAD = "llama2_7b_n32k"


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the bfloat16 bit patterns as uint16.  Inputs here are finite
    normal draws, so no NaN handling is needed; a non-finite input raises.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_bits_from_f32: non-finite input")
    u = x.view(np.uint32)
    # For finite inputs u + 0x8000 stays below 2^32, so uint32 cannot wrap.
    out = (u >> 16) & 1
    out += 0x7FFF
    out += u
    out >>= 16
    return out.astype(np.uint16)


def f64_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) exactly to float64."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# Operand variants of the same draws, for measuring how the matrix cores'
# throughput depends on the bits they multiply (the method is unchanged):
#   "normal"       the N(0,1) draws rounded to bfloat16 (every workload's data);
#   "mant2"        each bfloat16 value of q, k, v, dout keeps only the top 2 of
#                  its 7 stored mantissa bits (truncated toward zero);
#   "paired_keys"  in k and v, the rows at positions 64n+32 .. 64n+63 repeat the
#                  rows at 64n .. 64n+31, so the two 32-key halves of every
#                  64-key tile hold the same values.
OPERAND_VARIANTS = ("normal", "mant2", "paired_keys")


def make_inputs(B, N, H, Hkv, D, seed=0, with_dout=True, qk_prescale=None, operands="normal"):
    """Seeded bfloat16 inputs as uint16 bit arrays.

    ``qk_prescale`` (optional float) multiplies the float32 q and k draws
    before rounding; ``operands`` picks one of ``OPERAND_VARIANTS``.  Both
    change only the data, never the method.
    """
    if operands not in OPERAND_VARIANTS:
        raise ValueError(f"operands must be one of {OPERAND_VARIANTS}, not {operands!r}")
    rng = np.random.default_rng(seed)
    out = {}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv)):
        x = rng.standard_normal((B, N, heads, D), dtype=np.float32)
        if qk_prescale is not None and name in ("q", "k"):
            x = x * np.float32(qk_prescale)
        out[name] = bf16_bits_from_f32(x)
    if with_dout:
        out["dout"] = bf16_bits_from_f32(rng.standard_normal((B, N, H, D), dtype=np.float32))
    if operands == "mant2":
        for name in out:
            out[name] = out[name] & np.uint16(0xFFE0)
    elif operands == "paired_keys":
        for name in ("k", "v"):
            rows = np.arange((N // 64) * 64).reshape(-1, 64)[:, 32:].ravel()
            out[name][:, rows] = out[name][:, rows - 32]
    return out


def make_inputs_f32(B, N, H, Hkv, D, seed=0):
    """The same draws as ``make_inputs`` before rounding (float32 arrays)."""
    rng = np.random.default_rng(seed)
    return {name: rng.standard_normal((B, N, heads, D), dtype=np.float32)
            for name, heads in (("q", H), ("k", Hkv), ("v", Hkv))}


# LoRA-adapted q/k/v projections ahead of the attention path.  M = B * N
# token rows of the model width d_in; q has H * D output columns, k and v
# Hkv * D each; rank r within the 64-128 the "LoRA for Long-Context
# Adaptation" page recommends for long-context extension.
LORA_WORKLOADS = {
    "lora_qkv_tiny": dict(M=300, d_in=192, widths=(256, 128, 128), r=16, scale=1.0),
    "lora_qkv_llama2_7b_n32k": dict(M=32768, d_in=4096, widths=(4096, 4096, 4096), r=64, scale=1.0),
    "lora_qkv_llama2_70b_gqa_n32k": dict(M=32768, d_in=8192, widths=(8192, 1024, 1024), r=64, scale=1.0),
}

LORA_BENCH_WORKLOAD = "lora_qkv_llama2_7b_n32k"


def make_lora_inputs(M, d_in, widths, r, seed=0, with_dy=False):
    """Seeded bfloat16 inputs for the LoRA q/k/v projections (uint16 bits).

    Storage orientation (the one the library takes): x [M, d_in]; for each
    target p in (q, k, v): wt[p] [width_p, d_in] (the frozen weight, one row
    per output column), at[p] [r, d_in] (A transposed), bt[p] [width_p, r]
    (B transposed); dy[p] [M, width_p] when ``with_dy``.  Draw order: x, the
    three wt, the three at, the three bt, then the three dy, each
    ``standard_normal(float32)`` scaled before rounding: x and dy by 1,
    wt and at by 1/sqrt(d_in), bt by 1/sqrt(r), so every output column has
    unit-order magnitude (hidden states after RMSNorm, a trained adapter).
    """
    rng = np.random.default_rng(seed)

    def draw(shape, s):
        return bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(s))

    out = {"x": draw((M, d_in), 1.0)}
    out["wt"] = [draw((w, d_in), 1.0 / np.sqrt(d_in)) for w in widths]
    out["at"] = [draw((r, d_in), 1.0 / np.sqrt(d_in)) for _ in widths]
    out["bt"] = [draw((w, r), 1.0 / np.sqrt(max(r, 1))) for w in widths]
    if with_dy:
        out["dy"] = [draw((M, w), 1.0) for w in widths]
    return out
