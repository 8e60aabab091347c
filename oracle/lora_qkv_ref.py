"""Plain fp64 reference for the LoRA-adapted q/k/v projections ahead of S2-Attn.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Pages cited, by title:
  [Concept]  "LoRA for Long-Context Adaptation", praveentn.live concept note:
             "Why vanilla LoRA under-delivers on long context" (the two small
             trainable matrices A in R^{d x r} and B in R^{r x d} added to each
             frozen target projection, r << d) and "Practical recipe" (the
             targets are the attention projections, rank 64-128 for long
             context).
  [AIMech]   "LongLoRA and Shifted Sparse Attention (S^2-Attn)": LongLoRA
             trains low-rank adapters on the attention weights while the
             pretrained weights stay frozen.

What is computed.  The formula after the [Concept] sentence that introduces A
and B did not survive the text extraction.  The reading taken here is the
plainest one the surrounding text supports: with token activations as row
vectors x (one row per token), a frozen projection W in R^{d_in x d_out} and
the adapter pair A in R^{d_in x r}, B in R^{r x d_out},

    y = x W + s (x A) B,

i.e. the weight used is W + s A B.  The pages name no scale; ``s`` is an
argument (1 reproduces the bare "added to" reading; LoRA implementations
commonly pass alpha / r).  The three targets feeding attention are the q, k
and v projections, each with its own W, A, B; with grouped-query attention the
k and v outputs are narrower (Hkv * D columns) than q (H * D).

Backward (not on the pages: the calculus of the forward written out).  The
pretrained W is frozen, so the trainable gradients are those of A and B; the
input gradient is needed by the layers below.  With dy the gradient of y:
    dB = s (x A)^T dy,      dA = s x^T (dy B^T),
    dx = dy W^T + s (dy B^T) A^T,
summed over the q, k and v projections for dx.

All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np


def lora_projection(x, W, A, B, scale):
    """y = x W + s (x A) B for one target projection ([Concept] "Why vanilla
    LoRA under-delivers on long context": A and B added to the frozen W).

    x [M, d_in], W [d_in, d_out], A [d_in, r], B [r, d_out]; r may be 0.
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if x.shape[1] != W.shape[0] or A.shape[0] != W.shape[0] or B.shape[1] != W.shape[1] \
            or A.shape[1] != B.shape[0]:
        raise ValueError("lora_projection: shape mismatch")
    y = x @ W
    if A.shape[1] > 0:
        y = y + scale * ((x @ A) @ B)
    return y


def lora_qkv_forward(x, weights, adapters, scale):
    """The q, k and v projections of one attention layer, each LoRA-adapted.

    ``weights`` = (Wq, Wk, Wv), ``adapters`` = ((Aq, Bq), (Ak, Bk), (Av, Bv)),
    all in the page's orientation (see ``lora_projection``).  Returns the list
    [y_q, y_k, y_v]; the rows of y_q are the [N, H, D] query rows of the
    attention path once reshaped, likewise k and v with Hkv heads.
    """
    return [lora_projection(x, W, A, B, scale) for W, (A, B) in zip(weights, adapters)]


def lora_qkv_backward(x, weights, adapters, scale, dys):
    """Gradients of the three projections: returns (dx, [(dA, dB) per target]).

    dB = s (x A)^T dy and dA = s x^T (dy B^T) for each target; dx sums
    dy W^T + s (dy B^T) A^T over the three targets.  W is frozen (no dW).
    """
    x = np.asarray(x, dtype=np.float64)
    dx = np.zeros_like(x)
    grads = []
    for W, (A, B), dy in zip(weights, adapters, dys):
        W = np.asarray(W, dtype=np.float64)
        A = np.asarray(A, dtype=np.float64)
        B = np.asarray(B, dtype=np.float64)
        dy = np.asarray(dy, dtype=np.float64)
        xa = x @ A            # [M, r]
        dyb = dy @ B.T        # [M, r]
        dB = scale * (xa.T @ dy)
        dA = scale * (x.T @ dyb)
        dx += dy @ W.T + scale * (dyb @ A.T)
        grads.append((dA, dB))
    return dx, grads
