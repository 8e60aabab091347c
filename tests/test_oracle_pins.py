"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

None of these compares the oracle with itself.  Each pin is chosen so that a
plausible slip in the oracle (roll sign, group cut, mask direction, scale,
softmax normalisation, a dropped backward term, a transposed operand, the
GQA head map, the RoPE angle or direction) makes at least one test fail; the
mutation tests at the end plant such slips and check that the pins notice.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import s2attn_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, N, H, Hkv, D, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, N, H, D)), rng.standard_normal((B, N, Hkv, D)),
            rng.standard_normal((B, N, Hkv, D)), rng.standard_normal((B, N, H, D)))


# ---------------------------------------------------------------- roll / map

def test_roll_then_unroll_is_identity():
    x = _rand((37, 3), 1)
    for amt in (0, 1, 5, 36, 37, 100):
        assert np.array_equal(ref.roll_sequence(ref.roll_sequence(x, -amt), +amt), x)


def test_shift_worked_example_from_pages():
    gold = json.load(open(os.path.join(GOLDEN, "shift_worked_example.json")))
    N, G, sig = gold["N"], gold["G"], gold["shift"]
    shifted = ref.unit_positions(N, G, sig, 0)
    unshifted = ref.unit_positions(N, G, 0, 0)
    lo, hi = gold["shifted_first_group"]
    assert np.array_equal(shifted, np.arange(lo, hi + 1))
    lo, hi = gold["unshifted_first_group"]
    assert np.array_equal(unshifted, np.arange(lo, hi + 1))


def test_head_split_second_half_is_shifted():
    # Config "heads 2-3 shifted" of the tiny workload; the AIMech definition
    # shifts the second half of the heads.
    H = 4
    assert [ref.head_shift(h, H, 32) for h in range(H)] == [0, 0, 32, 32]


def test_wrap_group_is_circular():
    # Last group of a shifted head: last sigma tokens then the first sigma.
    N, G, sig = 16, 8, 4
    pos = ref.unit_positions(N, G, sig, N // G - 1)
    assert list(pos) == [12, 13, 14, 15, 0, 1, 2, 3]


def test_groups_partition_the_sequence():
    N, G = 48, 12
    for sig in (0, 1, 6, 11):
        allpos = np.concatenate([ref.unit_positions(N, G, sig, g) for g in range(N // G)])
        assert np.array_equal(np.sort(allpos), np.arange(N))


# ------------------------------------------------------------ forward values

def test_full_group_no_shift_equals_direct_causal_attention():
    B, N, H, D = 1, 12, 2, 8
    q, k, v, _ = _qkv(B, N, H, H, D, seed=2)
    out, lse = oracle.s2attn_forward(q, k, v, G=N, shift=0)
    for h in range(H):
        o_ref, l_ref = ref.dense_causal_attention(q[0, :, h], k[0, :, h], v[0, :, h])
        assert np.max(np.abs(out[0, :, h] - o_ref)) < 1e-12
        assert np.max(np.abs(lse[0, h] - l_ref)) < 1e-12


def test_full_group_no_shift_equals_torch_sdpa():
    B, N, H, D = 2, 64, 3, 16
    q, k, v, _ = _qkv(B, N, H, H, D, seed=3)
    out, _ = oracle.s2attn_forward(q, k, v, G=N, shift=0)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    o_t = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    assert np.max(np.abs(out - o_t.permute(0, 2, 1, 3).numpy())) < 1e-12


def test_no_shift_groups_are_block_diagonal_causal():
    B, N, H, D, G = 1, 48, 2, 8, 12
    q, k, v, _ = _qkv(B, N, H, H, D, seed=4)
    out, _ = oracle.s2attn_forward(q, k, v, G=G, shift=0)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    for g in range(N // G):
        sl = slice(g * G, (g + 1) * G)
        o_t = F.scaled_dot_product_attention(t(q[:, sl]), t(k[:, sl]), t(v[:, sl]), is_causal=True)
        assert np.max(np.abs(out[:, sl] - o_t.permute(0, 2, 1, 3).numpy())) < 1e-12


@pytest.mark.parametrize("N,G,shift,H,Hkv,D", [
    (16, 8, 4, 4, 4, 8),
    (16, 8, 4, 4, 2, 8),
    (16, 8, 3, 4, 2, 8),
    (24, 6, 5, 6, 2, 4),
    (256, 64, 32, 4, 4, 64),   # the tiny workload's shape
])
def test_brute_force_mask_agrees(N, G, shift, H, Hkv, D):
    q, k, v, _ = _qkv(1, N, H, Hkv, D, seed=N + G + shift)
    out, lse = oracle.s2attn_forward(q, k, v, G, shift)
    o_bf, l_bf = ref.brute_force_masked_attention(q, k, v, G, shift)
    assert np.max(np.abs(out - o_bf)) < 1e-12
    assert np.max(np.abs(lse - l_bf)) < 1e-12


def test_first_row_of_each_group_is_its_own_value():
    N, G, sig, H, D = 32, 8, 4, 4, 8
    q, k, v, _ = _qkv(1, N, H, H, D, seed=5)
    out, lse = oracle.s2attn_forward(q, k, v, G, sig)
    c = 1 / math.sqrt(D)
    for h in range(H):
        s = ref.head_shift(h, H, sig)
        for g in range(N // G):
            p0 = (g * G + s) % N          # first token of the group
            assert np.allclose(out[0, p0, h], v[0, p0, h], atol=1e-14, rtol=0)
            assert abs(lse[0, h, p0] - c * q[0, p0, h] @ k[0, p0, h]) < 1e-13


def test_wrap_group_leaks_across_the_sequence_end():
    # Circular reading: token 0 of a shifted head attends to tokens N-sigma..N-1.
    N, G, sig, H, D = 16, 8, 4, 2, 4
    q, k, v, _ = _qkv(1, N, H, H, D, seed=6)
    out, _ = oracle.s2attn_forward(q, k, v, G, sig)
    assert np.allclose(out[0, 0, 0], v[0, 0, 0])       # unshifted head: row 0 of group 0
    assert not np.allclose(out[0, 0, 1], v[0, 0, 1])   # shifted head: mid-group
    # and it equals causal attention over tokens 12..15, 0
    idx = [12, 13, 14, 15, 0]
    o_ref, _ = ref.dense_causal_attention(q[0, idx, 1], k[0, idx, 1], v[0, idx, 1])
    assert np.max(np.abs(out[0, 0, 1] - o_ref[-1])) < 1e-12


def test_softmax_rows_sum_to_one_via_lse():
    N, G, sig, H, Hkv, D = 32, 16, 8, 4, 2, 8
    q, k, v, _ = _qkv(1, N, H, Hkv, D, seed=7)
    _, lse = oracle.s2attn_forward(q, k, v, G, sig)
    c = 1 / math.sqrt(D)
    for h in range(H):
        kvh = ref.kv_head(h, H, Hkv)
        rho = (np.arange(N) - ref.head_shift(h, H, sig)) % N
        for p in range(N):
            allowed = (rho // G == rho[p] // G) & (rho <= rho[p])
            w = np.exp(c * k[0, allowed, kvh] @ q[0, p, h] - lse[0, h, p])
            assert abs(w.sum() - 1.0) < 1e-12


def test_constant_values_pass_through():
    N, G, sig, H, D = 32, 8, 4, 4, 8
    q, k, _, _ = _qkv(1, N, H, H, D, seed=8)
    v = np.ones((1, N, H, D)) * np.arange(D)
    out, _ = oracle.s2attn_forward(q, k, v, G, sig)
    assert np.max(np.abs(out - np.arange(D))) < 1e-12


def test_unit_rows_match_the_whole_forward():
    N, G, sig, H, Hkv, D = 32, 8, 4, 4, 2, 8
    q, k, v, _ = _qkv(1, N, H, Hkv, D, seed=9)
    rope = (10000.0, 2.0)
    out, lse = oracle.s2attn_forward(q, k, v, G, sig, rope=rope)
    for h in range(H):
        for g in range(N // G):
            pos, o, l = oracle.s2attn_unit_forward(q, k, v, G, sig, 0, h, g, rope=rope)
            assert np.max(np.abs(out[0, pos, h] - o)) < 1e-13
            assert np.max(np.abs(lse[0, h, pos] - l)) < 1e-13


def test_large_group_row_blocks_do_not_change_rows(monkeypatch):
    # Forcing many small row blocks must reproduce the single-block result.
    G, D = 40, 8
    q, k, v = _rand((G, D), 10), _rand((G, D), 11), _rand((G, D), 12)
    o1, l1 = ref.group_causal_attention(q, k, v, 0.3)
    monkeypatch.setattr(ref, "_BLOCK_BYTES", 8 * G * 3)
    o2, l2 = ref.group_causal_attention(q, k, v, 0.3)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14


# ------------------------------------------------------------------ backward

def _loss(q, k, v, w, G, sig, rope):
    out, _ = oracle.s2attn_forward(q, k, v, G, sig, rope=rope)
    return float(np.sum(out * w))


@pytest.mark.parametrize("Hkv,rope", [(4, None), (2, None), (2, (100.0, 2.0))])
def test_backward_matches_central_differences(Hkv, rope):
    B, N, H, D, G, sig = 1, 8, 4, 4, 4, 2
    q, k, v, w = _qkv(B, N, H, Hkv, D, seed=20 + Hkv)
    dq, dk, dv = oracle.s2attn_backward(q, k, v, w, G, sig, rope=rope)
    eps = 1e-6
    for x, gx in ((q, dq), (k, dk), (v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            fp = _loss(q, k, v, w, G, sig, rope)
            x[idx] = keep - eps
            fm = _loss(q, k, v, w, G, sig, rope)
            x[idx] = keep
            num[idx] = (fp - fm) / (2 * eps)
        assert np.max(np.abs(num - gx)) < 1e-7


def _torch_s2attn(q, k, v, G, sig):
    """S2-Attn written with torch ops (roll, view into groups, causal SDPA)."""
    B, N, H, D = q.shape
    Hkv = k.shape[2]
    r = H // Hkv
    k = k.repeat_interleave(r, dim=2)
    v = v.repeat_interleave(r, dim=2)
    outs = []
    for h in range(H):
        s = sig if h >= H // 2 else 0
        qs, ks, vs = (torch.roll(x[:, :, h], -s, dims=1).reshape(B * N // G, 1, G, D)
                      for x in (q, k, v))
        o = F.scaled_dot_product_attention(qs, ks, vs, is_causal=True)
        outs.append(torch.roll(o.reshape(B, N, D), s, dims=1))
    return torch.stack(outs, dim=2)


@pytest.mark.parametrize("Hkv", [4, 2])
def test_backward_matches_torch_autograd(Hkv):
    B, N, H, D, G, sig = 2, 48, 4, 8, 16, 8
    q, k, v, w = _qkv(B, N, H, Hkv, D, seed=30 + Hkv)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    out_t = _torch_s2attn(tq, tk, tv, G, sig)
    out, _ = oracle.s2attn_forward(q, k, v, G, sig)
    assert np.max(np.abs(out - out_t.detach().numpy())) < 1e-12
    (out_t * torch.from_numpy(w)).sum().backward()
    dq, dk, dv = oracle.s2attn_backward(q, k, v, w, G, sig)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - t.grad.numpy())) < 1e-11


def test_backward_group_invariants():
    # Per (k/v head, group): dS rows sum to 0, so sum_j dK_j = 0; P rows sum
    # to 1, so sum_j dV_j = sum_i dO_i over the q heads sharing the k/v head.
    B, N, H, Hkv, D, G, sig = 1, 32, 4, 2, 8, 8, 4
    q, k, v, w = _qkv(B, N, H, Hkv, D, seed=40)
    _, dk, dv = oracle.s2attn_backward(q, k, v, w, G, sig)
    for kvh in range(Hkv):
        hs = [h for h in range(H) if ref.kv_head(h, H, Hkv) == kvh]
        s = ref.head_shift(hs[0], H, sig)
        for g in range(N // G):
            pos = ref.unit_positions(N, G, s, g)
            assert np.max(np.abs(dk[0, pos, kvh].sum(0))) < 1e-11
            want = sum(w[0, pos, h].sum(0) for h in hs)
            assert np.max(np.abs(dv[0, pos, kvh].sum(0) - want)) < 1e-11


def test_unit_backward_sums_to_the_whole_backward():
    B, N, H, Hkv, D, G, sig = 1, 32, 4, 2, 8, 8, 4
    q, k, v, w = _qkv(B, N, H, Hkv, D, seed=41)
    rope = (10000.0, 4.0)
    dq, dk, dv = oracle.s2attn_backward(q, k, v, w, G, sig, rope=rope)
    acc_k = np.zeros_like(dk)
    acc_v = np.zeros_like(dv)
    for h in range(H):
        kvh = ref.kv_head(h, H, Hkv)
        for g in range(N // G):
            pos, uq, uk, uv = oracle.s2attn_unit_backward(q, k, v, w, G, sig, 0, h, g, rope=rope)
            assert np.max(np.abs(dq[0, pos, h] - uq)) < 1e-12
            acc_k[0, pos, kvh] += uk
            acc_v[0, pos, kvh] += uv
    assert np.max(np.abs(acc_k - dk)) < 1e-12 and np.max(np.abs(acc_v - dv)) < 1e-12


# ---------------------------------------------------------------------- GQA

def test_gqa_equals_mha_with_repeated_kv():
    B, N, H, Hkv, D, G, sig = 1, 32, 8, 2, 8, 8, 4
    q, k, v, w = _qkv(B, N, H, Hkv, D, seed=50)
    r = H // Hkv
    kr, vr = np.repeat(k, r, axis=2), np.repeat(v, r, axis=2)
    o1, l1 = oracle.s2attn_forward(q, k, v, G, sig)
    o2, l2 = oracle.s2attn_forward(q, kr, vr, G, sig)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13
    _, dk1, dv1 = oracle.s2attn_backward(q, k, v, w, G, sig)
    _, dk2, dv2 = oracle.s2attn_backward(q, kr, vr, w, G, sig)
    dk2 = dk2.reshape(B, N, Hkv, r, D).sum(3)
    dv2 = dv2.reshape(B, N, Hkv, r, D).sum(3)
    assert np.max(np.abs(dk1 - dk2)) < 1e-12 and np.max(np.abs(dv1 - dv2)) < 1e-12


# --------------------------------------------------------------------- RoPE

def test_rope_direction_and_angle_closed_form():
    # Pair 0 has frequency 1: at position p the angle is p / s radians,
    # counter-clockwise.  (1, 0) rotated by pi/2 is (0, 1).
    s = 4.0
    x = np.zeros((1, 2))
    x[0, 0] = 1.0
    y = ref.rope_rotate(x, np.array([s * math.pi / 2]), 10000.0, s)
    assert np.allclose(y, [[0.0, 1.0]], atol=1e-15)
    # Pair i of D has frequency base^(-2i/D): with base 16, D 4, pair 1 -> 1/4.
    ang = ref.rope_angles(np.array([8.0]), 4, 16.0, 2.0)
    assert np.allclose(ang, [[4.0, 1.0]], rtol=1e-15)


def test_rope_preserves_pair_norms_and_inverts():
    x = _rand((1, 20, 3, 16), 60)
    pos = np.arange(20)[None, :, None]
    y = ref.rope_rotate(x, pos, 10000.0, 8.0)
    n = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2
    assert np.max(np.abs(n(x) - n(y))) < 1e-12
    z = ref.rope_rotate(y, pos, 10000.0, 8.0, inverse=True)
    assert np.max(np.abs(z - x)) < 1e-13
    y0 = ref.rope_rotate(x[:, :1], np.zeros((1, 1, 1)), 10000.0, 8.0)
    assert np.array_equal(y0, x[:, :1])


def test_rope_logits_depend_only_on_relative_position():
    D = 16
    qv, kv = _rand((D,), 61), _rand((D,), 62)
    for s in (1.0, 8.0):
        def score(m, n):
            qm = ref.rope_rotate(qv[None], np.array([m]), 10000.0, s)[0]
            kn = ref.rope_rotate(kv[None], np.array([n]), 10000.0, s)[0]
            return qm @ kn
        for m, n, t in ((5, 2, 100), (700, 650, 3000), (9, 9, 77)):
            assert abs(score(m, n) - score(m + t, n + t)) < 1e-9


def test_position_interpolation_divides_positions():
    a = ref.rope_angles(np.arange(64), 32, 10000.0, 8.0)
    b = ref.rope_angles(np.arange(64) / 8.0, 32, 10000.0, 1.0)
    assert np.max(np.abs(a - b)) < 1e-13


def test_rope_applies_before_the_roll():
    # A token's rotation follows its original position, whichever group the
    # roll puts it in: rotating the rolled sequence by the rolled positions
    # equals rolling the rotated sequence.
    N, D, sig = 16, 8, 4
    x = _rand((N, D), 63)
    a = ref.roll_sequence(ref.rope_rotate(x, np.arange(N), 100.0, 2.0), -sig)
    b = ref.rope_rotate(ref.roll_sequence(x, -sig), ref.roll_sequence(np.arange(N), -sig), 100.0, 2.0)
    assert np.max(np.abs(a - b)) < 1e-14


# ------------------------------------------------------------ argument rules

@pytest.mark.parametrize("N,G,shift,H,Hkv", [
    (16, 5, 2, 4, 4),    # N not a multiple of G
    (16, 8, 8, 4, 4),    # shift out of [0, G)
    (16, 8, -1, 4, 4),
    (16, 8, 4, 3, 3),    # odd head count with a shift
    (16, 8, 4, 4, 1),    # odd k/v head count with a shift
    (16, 8, 0, 4, 3),    # H not a multiple of Hkv
])
def test_oracle_rejects_bad_arguments(N, G, shift, H, Hkv):
    q = np.zeros((1, N, H, 4))
    k = np.zeros((1, N, Hkv, 4))
    with pytest.raises(ValueError):
        oracle.s2attn_forward(q, k, k, G, shift)


# ------------------------------------------- pins notice planted mistakes

def _planted(monkeypatch, name, fn):
    monkeypatch.setattr(ref, name, fn)


def test_pins_catch_a_wrong_roll_sign(monkeypatch):
    _planted(monkeypatch, "roll_sequence", lambda x, a: np.roll(x, -a, axis=0))
    with pytest.raises(AssertionError):
        test_shift_worked_example_from_pages()


def test_pins_catch_a_missing_scale(monkeypatch):
    orig = ref.group_causal_attention
    _planted(monkeypatch, "group_causal_attention", lambda q, k, v, s: orig(q, k, v, 1.0))
    with pytest.raises(AssertionError):
        test_full_group_no_shift_equals_torch_sdpa()


def test_pins_catch_a_dropped_delta_term(monkeypatch):
    def bad(qg, kg, vg, dog, scale):
        G = qg.shape[0]
        s = scale * (qg @ kg.T)
        s = np.where(np.arange(G)[None] <= np.arange(G)[:, None], s, -np.inf)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        ds = p * (dog @ vg.T)                   # Delta dropped
        return scale * ds @ kg, scale * ds.T @ qg, p.T @ dog
    _planted(monkeypatch, "group_causal_attention_backward", bad)
    with pytest.raises(AssertionError):
        test_backward_matches_torch_autograd(2)


def test_pins_catch_a_wrong_kv_head_map(monkeypatch):
    _planted(monkeypatch, "kv_head", lambda h, H, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        test_backward_matches_torch_autograd(2)


def test_pins_catch_a_reversed_rotation(monkeypatch):
    orig = ref.rope_angles
    _planted(monkeypatch, "rope_angles", lambda p, D, b, s: -orig(p, D, b, s))
    with pytest.raises(AssertionError):
        test_rope_direction_and_angle_closed_form()


# ---------------------------------------------------------------------------
# Alternate-head shifting ("LoRA for Long-Context Adaptation", section
# "Shifted sparse attention": heads 1, 3, 5, ... shifted)
# ---------------------------------------------------------------------------

def test_alternate_pattern_shifts_the_odd_heads():
    assert [ref.head_shift(h, 4, 32, "alternate") for h in range(4)] == [0, 32, 0, 32]
    # Grouped-query sharing: the q heads of the odd k/v heads (two q heads each).
    assert [ref.head_shift(h, 8, 8, "alternate", 4) for h in range(8)] == [0, 0, 8, 8, 0, 0, 8, 8]
    with pytest.raises(ValueError):
        ref.head_shift(0, 4, 32, "every_third")


def test_alternate_pattern_worked_example():
    # The page's illustration: G = 2048, heads 1, 3, 5, ... shifted by 1024
    # cover tokens 1024 ... 3071 in their first group; heads 0, 2, 4 cover
    # 0 ... 2047.
    N, G = 8192, 2048
    for h in (1, 3, 5):
        pos = ref.unit_positions(N, G, ref.head_shift(h, 8, G // 2, "alternate"), 0)
        assert np.array_equal(pos, np.arange(1024, 3072))
    for h in (0, 2, 4):
        pos = ref.unit_positions(N, G, ref.head_shift(h, 8, G // 2, "alternate"), 0)
        assert np.array_equal(pos, np.arange(0, 2048))


def _half_order(H, Hkv):
    """q and k/v head orders that move the alternate pattern's shifted heads
    (the odd k/v heads and their q heads) into the second half."""
    r = H // Hkv
    kv = [j for j in range(Hkv) if j % 2 == 0] + [j for j in range(Hkv) if j % 2 == 1]
    qh = [j * r + i for j in kv for i in range(r)]
    return np.array(qh), np.array(kv)


@pytest.mark.parametrize("N,G,shift,H,Hkv,D", [(32, 8, 4, 4, 4, 8), (32, 8, 4, 8, 4, 8), (24, 6, 3, 4, 2, 4)])
def test_alternate_pattern_is_the_half_pattern_on_reordered_heads(N, G, shift, H, Hkv, D):
    # Heads are independent, so shifting the odd heads equals shifting the
    # second half after reordering the heads so the odd ones come last.
    q, k, v, do = _qkv(1, N, H, Hkv, D, seed=11 + H + Hkv)
    qo, ko = _half_order(H, Hkv)
    out_a, lse_a = oracle.s2attn_forward(q, k, v, G, shift, head_pattern="alternate")
    out_h, lse_h = oracle.s2attn_forward(q[:, :, qo], k[:, :, ko], v[:, :, ko], G, shift)
    assert np.max(np.abs(out_a[:, :, qo] - out_h)) < 1e-12
    assert np.max(np.abs(lse_a[:, qo] - lse_h)) < 1e-12
    dq_a, dk_a, dv_a = oracle.s2attn_backward(q, k, v, do, G, shift, head_pattern="alternate")
    dq_h, dk_h, dv_h = oracle.s2attn_backward(q[:, :, qo], k[:, :, ko], v[:, :, ko], do[:, :, qo], G, shift)
    assert np.max(np.abs(dq_a[:, :, qo] - dq_h)) < 1e-12
    assert np.max(np.abs(dk_a[:, :, ko] - dk_h)) < 1e-12
    assert np.max(np.abs(dv_a[:, :, ko] - dv_h)) < 1e-12


@pytest.mark.parametrize("N,G,shift,H,Hkv,D", [(16, 8, 4, 4, 4, 8), (24, 6, 5, 6, 2, 4), (16, 8, 4, 3, 3, 8)])
def test_alternate_pattern_brute_force_mask_agrees(N, G, shift, H, Hkv, D):
    q, k, v, _ = _qkv(1, N, H, Hkv, D, seed=3 * N + G)
    out, lse = oracle.s2attn_forward(q, k, v, G, shift, head_pattern="alternate")
    o_bf, l_bf = ref.brute_force_masked_attention(q, k, v, G, shift, head_pattern="alternate")
    assert np.max(np.abs(out - o_bf)) < 1e-12
    assert np.max(np.abs(lse - l_bf)) < 1e-12
