"""Plain, slow, fp64 reference for Shifted Sparse Attention (S2-Attn).

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Pages cited, by title:
  [AIMech]   "LongLoRA and Shifted Sparse Attention (S^2-Attn)", AIMech curated
             concept page.
  [Guide]    "LongLoRA: Efficient 100k Context LLM Fine-Tuning Guide", aifetchly
             blog.
  [Concept]  "LoRA for Long-Context Adaptation", praveentn.live concept note.
  [Abstract] "LongLoRA: Efficient Fine-tuning of Long-Context Large Language
             Models", arXiv abstract on the mlsanity index page.

What is computed (the AIMech opening definition): the projected q, k, v of
shape [B, N, H, D] are split along the head axis into two equal halves; the
second half is rolled by -G/2 along the sequence axis; the sequence is cut into
N/G groups of G tokens folded into the batch; standard (causal, per [Guide]
"How Shifted Short Attention Works") softmax attention with the 1/sqrt(D)
logit scale runs inside every group; the second half's output is rolled back
by +G/2 and the heads are concatenated again.

Readings taken where the pages leave a step open (each is also listed in the
design notes of the repository):
  * The roll is circular, as in [Guide] Step 1's sequence roll; the last
    shifted group therefore holds the last G/2 tokens followed by the first
    G/2, and causality is taken in that rolled order.
  * ``shift`` is an argument (the pages fix it to G/2); 0 <= shift < G.
  * Grouped-query attention: q head h reads k/v head floor(h / (H / Hkv)) and
    that k/v head is rolled by q head h's own shift.
  * The saved log-sum-exp is the natural log, indexed by original position.
  * RoPE ([Concept] "Why vanilla LoRA under-delivers"; linear position
    interpolation from [Concept] "Position interpolation"): the pair
    (x[2i], x[2i+1]) at original position p is rotated counter-clockwise by
    (p / s) * base^(-2i/D), before the roll.
  * The backward pass is not on the pages; it is the calculus of the forward
    definition written out (softmax Jacobian, adjoint of a permutation is its
    inverse, chain rule through the rotation).

All arithmetic is float64.  Large groups are processed a block of whole rows
at a time; every row's softmax still sees all of its row.
"""
from __future__ import annotations

import math

import numpy as np

# Rows per block when a group's G x G score matrix is formed; keeps one block
# of float64 scores under about 256 MiB.
_BLOCK_BYTES = 256 << 20


def _row_block(G: int) -> int:
    return max(1, min(G, _BLOCK_BYTES // (8 * max(G, 1))))


# ---------------------------------------------------------------------------
# Head split and the roll
# ---------------------------------------------------------------------------

HEAD_PATTERNS = ("second_half", "alternate")


def head_shift(h: int, H: int, shift: int, pattern: str = "second_half", Hkv: int | None = None) -> int:
    """Shift applied to head ``h``.

    "second_half": the second half of the heads (h >= H/2) is shifted, the
    first half is not ([AIMech] opening definition; [Guide] "1. Head
    Splitting into Standard and Shifted Groups").
    "alternate": alternate heads are shifted, heads 1, 3, 5, ... in the
    illustration of [Concept] "Shifted sparse attention".  With grouped-query
    sharing (Hkv < H) it is read as the q heads of the odd k/v heads, which
    is the odd heads when Hkv = H.
    """
    if pattern == "second_half":
        return int(shift) if h >= H // 2 else 0
    if pattern == "alternate":
        r = H // (Hkv if Hkv else H)
        return int(shift) if (h // r) % 2 == 1 else 0
    raise ValueError(f"unknown head pattern {pattern!r}")


def kv_head(h: int, H: int, Hkv: int) -> int:
    """k/v head read by q head ``h`` under grouped-query sharing (a reading:
    contiguous blocks of H/Hkv q heads share one k/v head)."""
    return h // (H // Hkv)


def roll_sequence(x: np.ndarray, amount: int) -> np.ndarray:
    """Circular roll of a per-head sequence ([N, ...], sequence on axis 0):
    ``out[i] = x[(i - amount) mod N]``.  ``amount = -G/2`` is the forward shift
    of the AIMech definition, ``+G/2`` shifts the outputs back."""
    return np.roll(x, amount, axis=0)


def unit_positions(N: int, G: int, shift_h: int, g: int) -> np.ndarray:
    """Original sequence positions of the G rows of group ``g`` of a head with
    shift ``shift_h``, obtained by applying the oracle's own roll to the index
    vector 0..N-1 and cutting group ``g`` out of it."""
    idx = roll_sequence(np.arange(N), -shift_h)
    return idx.reshape(N // G, G)[g].copy()


# ---------------------------------------------------------------------------
# RoPE with linear position interpolation
# ---------------------------------------------------------------------------

def rope_angles(positions, D: int, base: float, pos_scale: float) -> np.ndarray:
    """Angle of pair i at position p: (p / s) * base^(-2i/D).

    The frequency falls geometrically with the pair index ([Concept] "Why
    vanilla LoRA under-delivers on long context"); linear position
    interpolation divides the position by s = L_new / L_orig ([Concept]
    "Position interpolation: the prerequisite").  Returns an array of shape
    ``positions.shape + (D/2,)``.
    """
    p = np.asarray(positions, dtype=np.float64)
    i = np.arange(D // 2, dtype=np.float64)
    theta = np.float64(base) ** (-2.0 * i / D)
    return (p / np.float64(pos_scale))[..., None] * theta


def rope_rotate(x: np.ndarray, positions, base: float, pos_scale: float,
                inverse: bool = False) -> np.ndarray:
    """Rotate every adjacent pair (x[..., 2i], x[..., 2i+1]) by its angle.

    ``positions`` must broadcast against ``x[..., 0]``.  ``inverse=True``
    rotates by the negative angle (the transpose of the rotation, used for the
    gradient).
    """
    D = x.shape[-1]
    phi = rope_angles(positions, D, base, pos_scale)
    if inverse:
        phi = -phi
    c, s = np.cos(phi), np.sin(phi)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape), dtype=np.float64)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# ---------------------------------------------------------------------------
# Causal softmax attention inside one group
# ---------------------------------------------------------------------------

def group_causal_attention(qg, kg, vg, scale):
    """Causal softmax attention over the G rows of one group.

    S = scale * Q K^T with S[i, j] excluded for j > i ([Guide] "How Shifted
    Short Attention Works": standard causal self-attention in each group;
    Step 1's scaled dot product with the causal mask); P = max-subtracted
    softmax of each row over its allowed entries; O = P V;
    lse[i] = ln sum_{j<=i} exp(S[i, j]).
    Returns (O [G, D], lse [G]).
    """
    G = qg.shape[0]
    o = np.empty((G, vg.shape[1]), dtype=np.float64)
    lse = np.empty(G, dtype=np.float64)
    cols = np.arange(G)[None, :]
    blk = _row_block(G)
    for r0 in range(0, G, blk):
        r1 = min(G, r0 + blk)
        rows = np.arange(r0, r1)[:, None]
        s = scale * (qg[r0:r1] @ kg.T)
        s = np.where(cols <= rows, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        p = e / z
        o[r0:r1] = p @ vg
        lse[r0:r1] = (m + np.log(z))[:, 0]
    return o, lse


def group_causal_attention_backward(qg, kg, vg, dog, scale):
    """Gradients of ``group_causal_attention``'s O for the upstream dO.

    With P recomputed from the forward definition:
      dV = P^T dO;  dP = dO V^T;  Delta_i = sum_j P[i, j] dP[i, j];
      dS = P * (dP - Delta);  dQ = scale * dS K;  dK = scale * dS^T Q.
    Returns (dQ, dK, dV), each [G, D].
    """
    G = qg.shape[0]
    dq = np.empty_like(qg, dtype=np.float64)
    dk = np.zeros_like(kg, dtype=np.float64)
    dv = np.zeros_like(vg, dtype=np.float64)
    cols = np.arange(G)[None, :]
    blk = _row_block(G)
    for r0 in range(0, G, blk):
        r1 = min(G, r0 + blk)
        rows = np.arange(r0, r1)[:, None]
        s = scale * (qg[r0:r1] @ kg.T)
        s = np.where(cols <= rows, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        dp = dog[r0:r1] @ vg.T
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dv += p.T @ dog[r0:r1]
        dq[r0:r1] = scale * (ds @ kg)
        dk += scale * (ds.T @ qg[r0:r1])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Whole S2-Attn forward and backward
# ---------------------------------------------------------------------------

def _check(q, k, G, shift, head_pattern="second_half"):
    B, N, H, D = q.shape
    Hkv = k.shape[2]
    if G <= 0 or N % G != 0:
        raise ValueError("N must be a multiple of G")
    if not (0 <= shift < G):
        raise ValueError("shift must lie in [0, G)")
    if H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    if head_pattern == "second_half" and shift > 0 and (H % 2 != 0 or Hkv % 2 != 0):
        raise ValueError("a shifted half needs an even number of q and k/v heads")
    return B, N, H, Hkv, D


def _rotated(q, k, rope):
    if rope is None:
        return q, k
    base, s = rope
    pos = np.arange(q.shape[1])[None, :, None]
    return rope_rotate(q, pos, base, s), rope_rotate(k, pos, base, s)


def s2attn_forward(q, k, v, G, shift, rope=None, head_pattern="second_half"):
    """S2-Attn forward on float64 arrays q [B,N,H,D], k/v [B,N,Hkv,D].

    Steps of the AIMech definition, in order: (optional RoPE at the original
    positions), roll the shifted heads by -shift, reshape into N/G groups,
    causal attention per group, reshape back, roll the shifted heads' output
    by +shift.  Returns (out [B,N,H,D], lse [B,H,N]).
    """
    B, N, H, Hkv, D = _check(q, k, G, shift, head_pattern)
    qr, kr = _rotated(q, k, rope)
    scale = 1.0 / math.sqrt(D)
    NG = N // G
    out = np.empty((B, N, H, D), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            sig = head_shift(h, H, shift, head_pattern, Hkv)
            kvh = kv_head(h, H, Hkv)
            qh = roll_sequence(qr[b, :, h, :], -sig).reshape(NG, G, D)
            kh = roll_sequence(kr[b, :, kvh, :], -sig).reshape(NG, G, D)
            vh = roll_sequence(v[b, :, kvh, :], -sig).reshape(NG, G, D)
            oh = np.empty((NG, G, D))
            lh = np.empty((NG, G))
            for g in range(NG):
                oh[g], lh[g] = group_causal_attention(qh[g], kh[g], vh[g], scale)
            out[b, :, h, :] = roll_sequence(oh.reshape(N, D), +sig)
            lse[b, h, :] = roll_sequence(lh.reshape(N), +sig)
    return out, lse


def s2attn_backward(q, k, v, dout, G, shift, rope=None, head_pattern="second_half"):
    """Gradients of ``s2attn_forward``'s output w.r.t. q, k, v for the upstream
    gradient ``dout`` [B,N,H,D].

    dout is rolled like the forward input (the adjoint of the output roll-back
    is the forward roll), each group is differentiated, the group gradients
    are rolled back by +shift, k/v gradients of q heads sharing a k/v head are
    summed, and with RoPE the gradients of q and k pass back through the
    transposed rotation.  Returns (dq, dk, dv) with the input shapes.
    """
    B, N, H, Hkv, D = _check(q, k, G, shift, head_pattern)
    qr, kr = _rotated(q, k, rope)
    scale = 1.0 / math.sqrt(D)
    NG = N // G
    dq = np.empty((B, N, H, D), dtype=np.float64)
    dk = np.zeros((B, N, Hkv, D), dtype=np.float64)
    dv = np.zeros((B, N, Hkv, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            sig = head_shift(h, H, shift, head_pattern, Hkv)
            kvh = kv_head(h, H, Hkv)
            qh = roll_sequence(qr[b, :, h, :], -sig).reshape(NG, G, D)
            kh = roll_sequence(kr[b, :, kvh, :], -sig).reshape(NG, G, D)
            vh = roll_sequence(v[b, :, kvh, :], -sig).reshape(NG, G, D)
            doh = roll_sequence(dout[b, :, h, :], -sig).reshape(NG, G, D)
            dqh = np.empty((NG, G, D))
            dkh = np.empty((NG, G, D))
            dvh = np.empty((NG, G, D))
            for g in range(NG):
                dqh[g], dkh[g], dvh[g] = group_causal_attention_backward(
                    qh[g], kh[g], vh[g], doh[g], scale)
            dq[b, :, h, :] = roll_sequence(dqh.reshape(N, D), +sig)
            dk[b, :, kvh, :] += roll_sequence(dkh.reshape(N, D), +sig)
            dv[b, :, kvh, :] += roll_sequence(dvh.reshape(N, D), +sig)
    if rope is not None:
        base, s = rope
        pos = np.arange(N)[None, :, None]
        dq = rope_rotate(dq, pos, base, s, inverse=True)
        dk = rope_rotate(dk, pos, base, s, inverse=True)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# One (batch, head, group) unit, for sampled checks at full size
# ---------------------------------------------------------------------------

def head_unit_forward(qh, kh, vh, G, shift_h, g, rope=None):
    """One unit from one head's sequences.

    qh is q head h as an [N, D] float64 sequence at original positions, kh and
    vh the k/v head it reads; shift_h is that head's shift (head_shift()) and
    g the group.  Applies the optional RoPE at the original positions, rolls
    by -shift_h, cuts group g out and runs causal attention on it.
    Returns (positions [G], out [G, D], lse [G]).
    """
    (qg, kg, vg), pos, scale = _head_unit_operands(qh, kh, vh, None, G, shift_h, g, rope)
    o, lse = group_causal_attention(qg, kg, vg, scale)
    return pos, o, lse


def head_unit_backward(qh, kh, vh, doh, G, shift_h, g, rope=None):
    """Gradient contributions of one unit from one head's sequences (see
    head_unit_forward); doh is the upstream gradient of q head h's output.
    Returns (positions [G], dq [G, D], dk [G, D], dv [G, D]); dk/dv are this
    q head's share of its k/v head's gradient; with RoPE, dq and dk are
    passed back through the rotation."""
    (qg, kg, vg, dog), pos, scale = _head_unit_operands(qh, kh, vh, doh, G, shift_h, g, rope)
    dq, dk, dv = group_causal_attention_backward(qg, kg, vg, dog, scale)
    if rope is not None:
        base, s = rope
        dq = rope_rotate(dq, pos, base, s, inverse=True)
        dk = rope_rotate(dk, pos, base, s, inverse=True)
    return pos, dq, dk, dv


def _head_unit_operands(qh, kh, vh, doh, G, shift_h, g, rope):
    N, D = qh.shape
    if G <= 0 or N % G != 0:
        raise ValueError("N must be a multiple of G")
    if rope is not None:
        base, s = rope
        pos = np.arange(N)
        qh = rope_rotate(qh, pos, base, s)
        kh = rope_rotate(kh, pos, base, s)
    sl = slice(g * G, (g + 1) * G)
    ops = [roll_sequence(x, -shift_h)[sl] for x in (qh, kh, vh)]
    if doh is not None:
        ops.append(roll_sequence(doh, -shift_h)[sl])
    return ops, unit_positions(N, G, shift_h, g), 1.0 / math.sqrt(D)


def s2attn_unit_forward(q, k, v, G, shift, b, h, g, rope=None):
    """Output rows of one unit (batch b, q head h, group g) of the whole
    tensors.  Returns (positions [G], out [G, D], lse [G]) where
    ``positions`` are the original sequence positions of the rows; these rows
    equal the matching rows of ``s2attn_forward``."""
    B, N, H, Hkv, D = _check(q, k, G, shift)
    kvh = kv_head(h, H, Hkv)
    return head_unit_forward(q[b, :, h, :], k[b, :, kvh, :], v[b, :, kvh, :], G,
                             head_shift(h, H, shift), g, rope)


def s2attn_unit_backward(q, k, v, dout, G, shift, b, h, g, rope=None):
    """Gradient contributions of one unit (batch b, q head h, group g) of the
    whole tensors.  Returns (positions [G], dq [G, D], dk [G, D], dv [G, D]):
    dq rows are final; dk/dv rows are q head h's share (the full gradient of
    k/v head kv_head(h) at those positions is the sum over its H/Hkv q
    heads).  With RoPE, dq and dk are already passed back through the
    rotation."""
    B, N, H, Hkv, D = _check(q, k, G, shift)
    kvh = kv_head(h, H, Hkv)
    return head_unit_backward(q[b, :, h, :], k[b, :, kvh, :], v[b, :, kvh, :], dout[b, :, h, :], G,
                              head_shift(h, H, shift), g, rope)


# ---------------------------------------------------------------------------
# Independent references used only to pin the above
# ---------------------------------------------------------------------------

def dense_causal_attention(q, k, v):
    """Full causal softmax attention of one head, written as direct loops.

    q, k, v: [N, D] float64.  Row i attends to keys 0..i with logits
    q_i . k_j / sqrt(D).  Returns (out [N, D], lse [N]).  For tiny N only.
    """
    N, D = q.shape
    c = 1.0 / math.sqrt(D)
    out = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for i in range(N):
        logits = [c * float(np.dot(q[i], k[j])) for j in range(i + 1)]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = math.fsum(w)
        for j in range(i + 1):
            out[i] += (w[j] / z) * v[j]
        lse[i] = mx + math.log(z)
    return out, lse


def brute_force_masked_attention(q, k, v, G, shift, head_pattern="second_half"):
    """S2-Attn as dense N x N attention under an explicit mask; no roll and no
    reshape.  Token p of a head with shift sigma sits at rolled index
    rho(p) = (p - sigma) mod N; p may attend to p' exactly when both fall in
    the same group (floor(rho/G) equal) and rho(p') <= rho(p).
    Returns (out [B,N,H,D], lse [B,H,N]).  For tiny N only.
    """
    B, N, H, Hkv, D = _check(q, k, G, shift, head_pattern)
    c = 1.0 / math.sqrt(D)
    out = np.empty((B, N, H, D))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            sig = head_shift(h, H, shift, head_pattern, Hkv)
            kvh = kv_head(h, H, Hkv)
            rho = (np.arange(N) - sig) % N
            grp = rho // G
            allowed = (grp[:, None] == grp[None, :]) & (rho[None, :] <= rho[:, None])
            s = c * (q[b, :, h, :] @ k[b, :, kvh, :].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            out[b, :, h, :] = (e / z) @ v[b, :, kvh, :]
            lse[b, h, :] = (m + np.log(z))[:, 0]
    return out, lse
