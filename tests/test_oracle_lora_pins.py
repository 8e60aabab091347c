"""Pins for the fp64 LoRA q/k/v projection oracle (CPU only).

Each pin checks the oracle against something other than itself: a hand-worked
instance, brute-force loops on tiny inputs, the reduction to a plain linear
layer (a library routine) when the adapter is zero, the rank bound of the
low-rank update, the merged-weight identity, and for the backward exact
directional derivatives (the projection is linear in each of x, A and B) and
autograd.  The mutation tests at the end plant plausible slips in the oracle
(a dropped or subtracted update, a transposed weight, a misplaced scale, dropped backward
terms) and check that a pin fails.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import lora_qkv_ref as lref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mats(M, d_in, d_out, r, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, d_in)), rng.standard_normal((d_in, d_out)),
            rng.standard_normal((d_in, r)), rng.standard_normal((r, d_out)))


# ------------------------------------------------------------------- forward

def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "lora_worked_example.json")))
    y = lref.lora_projection(np.array(g["x"], float), np.array(g["W"], float), np.array(g["A"], float),
                             np.array(g["B"], float), g["scale"])
    assert np.array_equal(y, np.array(g["y"], float))


def test_brute_force_loops():
    # Shapes all distinct so that a transposed operand cannot line up.
    x, W, A, B = _mats(3, 5, 4, 2, 1)
    s = 0.75
    y = lref.lora_projection(x, W, A, B, s)
    for m in range(3):
        for o in range(4):
            base = sum(x[m, k] * W[k, o] for k in range(5))
            low = sum(sum(x[m, k] * A[k, j] for k in range(5)) * B[j, o] for j in range(2))
            assert abs(y[m, o] - (base + s * low)) < 1e-12


def test_zero_adapter_is_a_plain_linear_layer():
    x, W, A, B = _mats(7, 6, 5, 3, 2)
    want = F.linear(torch.from_numpy(x), torch.from_numpy(W.T.copy())).numpy()
    assert np.allclose(lref.lora_projection(x, W, A, np.zeros_like(B), 1.3), want, rtol=0, atol=1e-12)
    assert np.allclose(lref.lora_projection(x, W, A[:, :0], B[:0], 1.3), want, rtol=0, atol=1e-12)
    assert np.allclose(lref.lora_projection(x, W, A, B, 0.0), want, rtol=0, atol=1e-12)


def test_update_has_rank_at_most_r():
    x, W, A, B = _mats(40, 12, 10, 3, 3)
    y = lref.lora_projection(x, np.zeros_like(W), A, B, 1.0)
    sv = np.linalg.svd(y, compute_uv=False)
    assert sv[2] > 1e-3 * sv[0]          # the update is really there, rank r = 3
    assert sv[3] < 1e-10 * sv[0]         # and has rank no more than r


def test_merged_weight_identity():
    # The adapted layer acts as the single weight W + s A B.
    x, W, A, B = _mats(9, 8, 6, 2, 4)
    s = -1.7
    assert np.allclose(lref.lora_projection(x, W, A, B, s), x @ (W + s * (A @ B)), rtol=1e-12, atol=1e-12)


def test_scale_enters_linearly():
    x, W, A, B = _mats(4, 6, 5, 2, 5)
    y0 = lref.lora_projection(x, W, A, B, 0.0)
    y1 = lref.lora_projection(x, W, A, B, 1.0)
    y3 = lref.lora_projection(x, W, A, B, 3.0)
    assert np.allclose(y3 - y0, 3.0 * (y1 - y0), rtol=1e-12, atol=1e-12)


def test_qkv_targets_are_independent_and_gqa_widths():
    rng = np.random.default_rng(6)
    d, r = 8, 2
    widths = (8, 4, 4)  # grouped-query attention: k and v narrower than q
    x = rng.standard_normal((5, d))
    Ws = [rng.standard_normal((d, w)) for w in widths]
    ads = [(rng.standard_normal((d, r)), rng.standard_normal((r, w))) for w in widths]
    ys = lref.lora_qkv_forward(x, Ws, ads, 0.5)
    assert [y.shape for y in ys] == [(5, 8), (5, 4), (5, 4)]
    for y, W, (A, B) in zip(ys, Ws, ads):
        assert np.array_equal(y, lref.lora_projection(x, W, A, B, 0.5))


def test_shape_mismatch_raises():
    x, W, A, B = _mats(3, 5, 4, 2, 7)
    with pytest.raises(ValueError):
        lref.lora_projection(x, W, A, B.T, 1.0)


# ------------------------------------------------------------------ backward

def _loss(x, Ws, ads, s, dys):
    return sum(float(np.sum(dy * y)) for dy, y in zip(dys, lref.lora_qkv_forward(x, Ws, ads, s)))


def _problem(seed, M=6, d=5, widths=(4, 3, 3), r=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, d))
    Ws = [rng.standard_normal((d, w)) for w in widths]
    ads = [(rng.standard_normal((d, r)), rng.standard_normal((r, w))) for w in widths]
    dys = [rng.standard_normal((M, w)) for w in widths]
    return rng, x, Ws, ads, dys


def test_backward_exact_directional_derivatives():
    # L = sum <dy_p, y_p> is linear in x, and in each A_p and B_p separately,
    # so a central difference along any direction is exact up to rounding.
    rng, x, Ws, ads, dys = _problem(8)
    s = 1.25
    dx, grads = lref.lora_qkv_backward(x, Ws, ads, s, dys)
    e = rng.standard_normal(x.shape)
    fd = (_loss(x + e, Ws, ads, s, dys) - _loss(x - e, Ws, ads, s, dys)) / 2
    assert abs(fd - np.sum(dx * e)) < 1e-9 * (1 + abs(fd))
    for p in range(3):
        for which in (0, 1):
            e = rng.standard_normal(ads[p][which].shape)

            def moved(sign):
                new = [list(a) for a in ads]
                new[p][which] = ads[p][which] + sign * e
                return [tuple(a) for a in new]

            fd = (_loss(x, Ws, moved(+1), s, dys) - _loss(x, Ws, moved(-1), s, dys)) / 2
            assert abs(fd - np.sum(grads[p][which] * e)) < 1e-9 * (1 + abs(fd))


def test_backward_matches_autograd():
    _, x, Ws, ads, dys = _problem(9, M=7, d=6, widths=(6, 2, 2), r=3)
    s = 0.5
    tx = torch.tensor(x, requires_grad=True)
    tads = [(torch.tensor(A, requires_grad=True), torch.tensor(B, requires_grad=True)) for A, B in ads]
    loss = 0
    for W, (A, B), dy in zip(Ws, tads, dys):
        y = F.linear(tx, torch.tensor(W.T.copy())) + s * F.linear(F.linear(tx, A.T), B.T)
        loss = loss + (y * torch.tensor(dy)).sum()
    loss.backward()
    dx, grads = lref.lora_qkv_backward(x, Ws, ads, s, dys)
    assert np.allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-12)
    for (dA, dB), (A, B) in zip(grads, tads):
        assert np.allclose(dA, A.grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(dB, B.grad.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------- planted slips are caught

def _fails(fn):
    # A pin fails by an assertion or, for a shape slip, by raising.
    try:
        fn()
    except Exception:
        return True
    return False


def test_pins_catch_a_dropped_update(monkeypatch):
    monkeypatch.setattr(lref, "lora_projection", lambda x, W, A, B, s: np.asarray(x, float) @ W)
    assert _fails(test_worked_example) and _fails(test_brute_force_loops)


def test_pins_catch_a_transposed_weight(monkeypatch):
    def bad(x, W, A, B, s):
        x = np.asarray(x, float)
        return x @ np.asarray(W).T + s * ((x @ A) @ B)
    monkeypatch.setattr(lref, "lora_projection", bad)
    assert _fails(test_brute_force_loops) and _fails(test_worked_example)


def test_pins_catch_a_subtracted_update(monkeypatch):
    def bad(x, W, A, B, s):
        x = np.asarray(x, float)
        return x @ W - s * ((x @ A) @ B)
    monkeypatch.setattr(lref, "lora_projection", bad)
    assert _fails(test_brute_force_loops) and _fails(test_merged_weight_identity)


def test_pins_catch_a_misplaced_scale(monkeypatch):
    def bad(x, W, A, B, s):
        x = np.asarray(x, float)
        return s * (x @ W) + (x @ A) @ B
    monkeypatch.setattr(lref, "lora_projection", bad)
    assert _fails(test_worked_example) and _fails(test_zero_adapter_is_a_plain_linear_layer)


def test_pins_catch_a_dropped_backward_term(monkeypatch):
    orig = lref.lora_qkv_backward

    def bad(x, Ws, ads, s, dys):
        dx, grads = orig(x, Ws, ads, s, dys)
        # Drop the adapter's contribution to dx.
        for (A, B), dy in zip(ads, dys):
            dx = dx - s * ((np.asarray(dy) @ np.asarray(B).T) @ np.asarray(A).T)
        return dx, grads
    monkeypatch.setattr(lref, "lora_qkv_backward", bad)
    assert _fails(test_backward_exact_directional_derivatives) and _fails(test_backward_matches_autograd)


def test_pins_catch_a_missing_backward_scale(monkeypatch):
    orig = lref.lora_qkv_backward

    def bad(x, Ws, ads, s, dys):
        dx, grads = orig(x, Ws, ads, s, dys)
        return dx, [(dA / s, dB) for dA, dB in grads]
    monkeypatch.setattr(lref, "lora_qkv_backward", bad)
    assert _fails(test_backward_exact_directional_derivatives)
