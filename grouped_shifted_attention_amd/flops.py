"""FLOP and byte accounting of S2-Attn used by the benchmark.

Effective causal FLOPs: one unit (batch, head, group) computes the two G x G
x D products Q K^T and P V over the causal half, 2 * (G*G/2) * D * 2 = 2 G^2 D
FLOPs; over the N/G groups of every head that is 2 * B * H * N * G * D for
the forward.  The backward recomputes S and adds dP, dV, dK, dQ: counted as
2.5 times the forward.  The shift adds no FLOPs (AIMech "LongLoRA and Shifted
Sparse Attention (S^2-Attn)", claim on the half-group shift: N/G groups cut
attention FLOPs N/G-fold and the shift costs nothing extra).

Algorithmic bytes are the minimum HBM traffic of one call: every input read
once and every output written once.
"""


def s2attn_fwd_flops(B, H, N, G, D):
    return 2 * B * H * N * G * D


def s2attn_bwd_flops(B, H, N, G, D):
    return 5 * B * H * N * G * D


def fwd_algorithmic_bytes(B, N, H, Hkv, D):
    """q, k, v read; out written (bf16); lse written (fp32)."""
    return 2 * B * N * D * (2 * H + 2 * Hkv) + 4 * B * H * N


def bwd_algorithmic_bytes(B, N, H, Hkv, D):
    """q, k, v, out, dout read and dq, dk, dv written (bf16); lse read (fp32)."""
    return 2 * B * N * D * (4 * H + 4 * Hkv) + 4 * B * H * N
