"""GPU parity of the LoRA q/k/v projections against the fp64 oracle.

Small shapes compare every output element and the low-rank activations the
call leaves in its workspace; they span ragged token tiles (M not a multiple
of 256), ragged column tiles (widths not multiples of 256), odd and even
numbers of 64-deep reduction tiles, ranks that fill part of a reduction tile
(8, 16, 72), no adapter (r = 0), a single token, and grouped-query widths.
The full LLaMA2-7B and 70B projection shapes at 32k tokens, in the launch
configuration the benchmark times, compare sampled token rows (every column
of them, across the first, middle and last token tiles).

Tolerance, derived from the arithmetic (not fitted): with u = 2^-8 the bf16
unit roundoff and fp32 accumulation over n = d_in + r terms, each element
obeys
    |y_gpu - y| <= u |y| + u s (|x A| |B|) + n 2^-24 (|x| |W| + s |x A| |B|)
(output rounding, the bf16 rounding of the low-rank activations, and the
first-order bound of an n-term fp32 sum), evaluated per element from the
fp64 inputs with a 1% margin; in addition rel-L2 <= 1e-2 over each output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from grouped_shifted_attention_amd import ops
from gpu_helpers import to_f64, to_gpu
from workloads import f64_from_bf16_bits

pytestmark = pytest.mark.gpu

U = 2.0 ** -8
REL_L2 = 1e-2

# name, M, d_in, width_q, width_kv, r, scale
CASES = [
    ("tiny_ragged", 300, 192, 256, 128, 16, 1.0),
    ("rank8_one_ktile", 257, 64, 64, 64, 8, 1.0),
    ("rank72_two_tail_tiles", 512, 256, 384, 128, 72, 0.75),
    ("no_adapter", 300, 128, 192, 64, 0, 1.0),
    ("rank64_scale_half", 1000, 512, 512, 512, 64, 0.5),
    ("gqa_widths", 777, 1024, 1024, 128, 64, 2.0),
    ("single_token", 1, 128, 128, 64, 16, 1.0),
    ("rank128_multi_band", 2304, 320, 768, 256, 128, 1.0),
]
IDS = [c[0] for c in CASES]


def _inputs(M, d_in, wq, wkv, r, seed):
    d = workloads.make_lora_inputs(M, d_in, (wq, wkv, wkv), r, seed=seed)
    f = {"x": f64_from_bf16_bits(d["x"]),
         "wt": [f64_from_bf16_bits(w) for w in d["wt"]],
         "at": [f64_from_bf16_bits(a) for a in d["at"]],
         "bt": [f64_from_bf16_bits(b) for b in d["bt"]]}
    return d, f


def _call(d, r, scale):
    x = to_gpu(d["x"])
    wt = [to_gpu(w) for w in d["wt"]]
    at = [to_gpu(a) for a in d["at"]] if r > 0 else None
    bt = [to_gpu(b) for b in d["bt"]] if r > 0 else None
    q, k, v, ws = ops.s2attn_lora_qkv_fwd(x, wt, at, bt, scale)
    torch.cuda.synchronize()
    t = None
    if r > 0:
        t = ws[: x.shape[0] * 3 * r * 2].view(torch.bfloat16).view(x.shape[0], 3 * r)
    return [q, k, v], t


def _reference(f, rows, r, scale):
    """Oracle outputs on the given token rows, in the page's orientation."""
    x = f["x"][rows]
    Ws = [w.T for w in f["wt"]]
    ads = [(a.T, b.T) for a, b in zip(f["at"], f["bt"])] if r > 0 else \
        [(np.zeros((w.shape[1], 0)), np.zeros((0, w.shape[0]))) for w in f["wt"]]
    ys = oracle.lora_qkv_forward(x, Ws, ads, scale)
    # Elementwise bound of the derived tolerance.
    n = x.shape[1] + r
    bounds = []
    for y, W, (A, B) in zip(ys, Ws, ads):
        base = np.abs(x) @ np.abs(W)
        low = abs(scale) * (np.abs(x @ A) @ np.abs(B)) if r > 0 else 0.0
        bounds.append(1.01 * (U * np.abs(y) + U * low + n * 2.0 ** -24 * (base + low)) + 1e-30)
    t_ref = np.concatenate([scale * (x @ A) for A, _ in ads], axis=1) if r > 0 else None
    t_bound = None
    if r > 0:
        t_bound = 1.01 * (U * np.abs(t_ref) + x.shape[1] * 2.0 ** -24 * abs(scale) *
                          np.concatenate([np.abs(x) @ np.abs(A) for A, _ in ads], axis=1)) + 1e-30
    return ys, bounds, t_ref, t_bound


def _check(name, got, ref, bound):
    d = np.abs(got - ref)
    worst = float(np.max(d / bound)) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else 0.0
    print(f"  {name}: max |err|/bound {worst:.3f}, max |err| {float(d.max()) if d.size else 0:.3e}, "
          f"rel-L2 {rel:.2e}", flush=True)
    assert worst <= 1.0, f"{name}: error exceeds the derived bound ({worst:.3f} x)"
    assert rel <= REL_L2, f"{name}: rel-L2 {rel:.3e}"


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_lora_qkv_small(case):
    name, M, d_in, wq, wkv, r, scale = case
    d, f = _inputs(M, d_in, wq, wkv, r, seed=11)
    ys, t = _call(d, r, scale)
    rows = np.arange(M)
    refs, bounds, t_ref, t_bound = _reference(f, rows, r, scale)
    for nm, y, ref, b in zip(("q", "k", "v"), ys, refs, bounds):
        _check(nm, to_f64(y), ref, b)
    if r > 0:
        _check("x A (workspace)", to_f64(t), t_ref, t_bound)


def test_lora_qkv_deterministic_and_zero_adapter_equals_no_adapter():
    M, d_in, wq, wkv, r = 600, 256, 256, 128, 16
    d, _ = _inputs(M, d_in, wq, wkv, r, seed=12)
    y1, _ = _call(d, r, 1.0)
    y2, _ = _call(d, r, 1.0)
    for a, b in zip(y1, y2):
        assert torch.equal(a, b)
    # B = 0: the update vanishes exactly, so the result equals r = 0 bit for bit.
    dz = dict(d)
    dz["bt"] = [np.zeros_like(b) for b in d["bt"]]
    yz, _ = _call(dz, r, 1.0)
    y0, _ = _call(d, 0, 1.0)
    for a, b in zip(yz, y0):
        assert torch.equal(a, b)


@pytest.mark.parametrize("workload", ["lora_qkv_llama2_7b_n32k", "lora_qkv_llama2_70b_gqa_n32k"])
def test_lora_qkv_full_size_sampled_rows(workload):
    w = workloads.LORA_WORKLOADS[workload]
    M, d_in, (wq, wkv, _), r, scale = w["M"], w["d_in"], w["widths"], w["r"], w["scale"]
    d, f = _inputs(M, d_in, wq, wkv, r, seed=0)
    ys, t = _call(d, r, scale)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M // 2, M - 257, M - 1],
                                     rng.integers(0, M, 57)]))
    refs, bounds, t_ref, t_bound = _reference(f, rows, r, scale)
    idx = torch.from_numpy(rows).to("cuda:0")
    for nm, y, ref, b in zip(("q", "k", "v"), ys, refs, bounds):
        _check(nm, to_f64(y.index_select(0, idx)), ref, b)
    _check("x A (workspace)", to_f64(t.index_select(0, idx)), t_ref, t_bound)


# ------------------------------------------------------------------ backward
#
# Bar, derived like the forward's (u = 2^-8; an n-term fp32 sum is off by at
# most n 2^-24 times the sum of its absolute terms, first order).  With
# dTs = s dy B^T (exact), |dTs| its magnitude and S = s |dy| |B|^T the sum of
# the absolute terms that form it (width terms), each element obeys
#   dx  : u|dx| + u |dTs| |A| + width 2^-24 S |A| + n 2^-24 (|dy| |W| + |dTs| |A|),
#         n = sum(width) + 3r
#   dA^T: u|dA| + u |x|^T |dTs| + width 2^-24 |x|^T S + M 2^-24 |x|^T |dTs|
#   dB^T: u|dB| + (u + M 2^-24) |T|^T |dy| + d_in 2^-24 (s |x| |A|)^T |dy|,  T = s x A
# (the bf16 rounding of dTs and of the forward's T, the fp32 sums that form
# them, the final sums and the output rounding).

def _bwd_bounds(x, Ws, ads, dy, scale, rows=None):
    """Oracle gradients and their bounds; dx only on `rows` when given."""
    M, d_in = x.shape
    xr = x if rows is None else x[rows]
    n = sum(W.shape[1] for W in Ws) + 3 * ads[0][0].shape[1]
    dx = np.zeros((xr.shape[0], d_in))
    dxb = np.zeros_like(dx)
    out = {}
    for p, (W, (A, B), g) in enumerate(zip(Ws, ads, dy)):
        width = W.shape[1]
        gr = g if rows is None else g[rows]
        dts = scale * (gr @ B.T)
        S = abs(scale) * (np.abs(gr) @ np.abs(B).T)
        dx += gr @ W.T + dts @ A.T
        dxb += U * (np.abs(dts) @ np.abs(A).T) + width * 2.0 ** -24 * (S @ np.abs(A).T) \
            + n * 2.0 ** -24 * (np.abs(gr) @ np.abs(W).T + np.abs(dts) @ np.abs(A).T)
        if rows is None:
            dA = x.T @ dts
            ba = U * np.abs(dA) + (U + M * 2.0 ** -24) * (np.abs(x).T @ np.abs(dts)) \
                + width * 2.0 ** -24 * (np.abs(x).T @ S)
            T = scale * (x @ A)
            dB = T.T @ g
            bb = U * np.abs(dB) + (U + M * 2.0 ** -24) * (np.abs(T).T @ np.abs(g)) \
                + d_in * 2.0 ** -24 * ((abs(scale) * (np.abs(x) @ np.abs(A))).T @ np.abs(g))
            out[f"dA{p}"] = (dA.T, 1.01 * ba.T + 1e-30)
            out[f"dB{p}"] = (dB.T, 1.01 * bb.T + 1e-30)
    out["dx"] = (dx, 1.01 * (dxb + U * np.abs(dx)) + 1e-30)
    return out


def _bwd_call(d, r, scale):
    x = to_gpu(d["x"])
    wt = [to_gpu(w) for w in d["wt"]]
    at = [to_gpu(a) for a in d["at"]] if r > 0 else None
    bt = [to_gpu(b) for b in d["bt"]] if r > 0 else None
    dys = [to_gpu(g) for g in d["dy"]]
    _, _, _, ws = ops.s2attn_lora_qkv_fwd(x, wt, at, bt, scale)
    t = ws[: x.shape[0] * 3 * r * 2].view(torch.bfloat16).view(x.shape[0], 3 * r) if r > 0 else None
    dx, dat, dbt = ops.s2attn_lora_qkv_bwd(x, wt, at, bt, scale, t, dys)
    torch.cuda.synchronize()
    return dx, dat, dbt


BWD_CASES = [c for c in CASES if c[0] != "single_token"] + [("single_token_bwd", 1, 128, 128, 64, 16, 1.0)]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_lora_qkv_backward_small(case):
    name, M, d_in, wq, wkv, r, scale = case
    d = workloads.make_lora_inputs(M, d_in, (wq, wkv, wkv), r, seed=21, with_dy=True)
    f = {"x": f64_from_bf16_bits(d["x"]), "wt": [f64_from_bf16_bits(w) for w in d["wt"]],
         "at": [f64_from_bf16_bits(a) for a in d["at"]], "bt": [f64_from_bf16_bits(b) for b in d["bt"]]}
    dy = [f64_from_bf16_bits(g) for g in d["dy"]]
    dx, dat, dbt = _bwd_call(d, r, scale)
    if r == 0:
        assert dat is None and dbt is None
    # The oracle's own backward is the reference; the bounds come from the
    # same fp64 products.
    Ws = [w.T for w in f["wt"]]
    ads = [(a.T, b.T) for a, b in zip(f["at"], f["bt"])]  # r = 0: empty adapters
    ref_dx, ref_grads = oracle.lora_qkv_backward(f["x"], Ws, ads, scale, dy)
    ref = _bwd_bounds(f["x"], Ws, ads, dy, scale)
    assert np.allclose(ref["dx"][0], ref_dx, rtol=1e-10, atol=1e-10)
    _check("dx", to_f64(dx), ref_dx, ref["dx"][1])
    for p in range(3 if r > 0 else 0):
        _check(f"dA_{'qkv'[p]}^T", to_f64(dat[p]), ref_grads[p][0].T, ref[f"dA{p}"][1])
        _check(f"dB_{'qkv'[p]}^T", to_f64(dbt[p]), ref_grads[p][1].T, ref[f"dB{p}"][1])


def test_lora_qkv_backward_deterministic():
    M, d_in, wq, wkv, r = 3000, 256, 256, 128, 16
    d = workloads.make_lora_inputs(M, d_in, (wq, wkv, wkv), r, seed=22, with_dy=True)
    a = _bwd_call(d, r, 1.0)
    b = _bwd_call(d, r, 1.0)
    assert torch.equal(a[0], b[0])
    for p in range(3):
        assert torch.equal(a[1][p], b[1][p]) and torch.equal(a[2][p], b[2][p])


@pytest.mark.parametrize("workload", ["lora_qkv_llama2_7b_n32k"])
def test_lora_qkv_backward_full_size(workload):
    # dA and dB reduce over every token, so they are compared in full; dx on
    # sampled token rows.
    w = workloads.LORA_WORKLOADS[workload]
    M, d_in, (wq, wkv, _), r, scale = w["M"], w["d_in"], w["widths"], w["r"], w["scale"]
    d = workloads.make_lora_inputs(M, d_in, (wq, wkv, wkv), r, seed=0, with_dy=True)
    dx, dat, dbt = _bwd_call(d, r, scale)
    x = f64_from_bf16_bits(d["x"])
    Ws = [f64_from_bf16_bits(w_).T for w_ in d["wt"]]
    ads = [(f64_from_bf16_bits(a).T, f64_from_bf16_bits(b).T) for a, b in zip(d["at"], d["bt"])]
    dy = [f64_from_bf16_bits(g) for g in d["dy"]]
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 255, 256, M // 2, M - 1], rng.integers(0, M, 27)]))
    ref = _bwd_bounds(x, Ws, ads, dy, scale)          # dA, dB in full
    refx = _bwd_bounds(x, Ws, ads, dy, scale, rows)   # dx on the sampled rows
    # The oracle on the sampled rows agrees with the bound helper's products.
    ox, _ = oracle.lora_qkv_backward(x[rows], Ws, ads, scale, [g[rows] for g in dy])
    assert np.allclose(refx["dx"][0], ox, rtol=1e-10, atol=1e-10)
    for p in range(3):
        _check(f"dA_{'qkv'[p]}^T", to_f64(dat[p]), *ref[f"dA{p}"])
        _check(f"dB_{'qkv'[p]}^T", to_f64(dbt[p]), *ref[f"dB{p}"])
    idx = torch.from_numpy(rows).to("cuda:0")
    _check("dx (sampled rows)", to_f64(dx.index_select(0, idx)), *refx["dx"])
