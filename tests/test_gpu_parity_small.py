"""GPU parity against the fp64 oracle on shapes the oracle finishes in seconds.

Every element of out, lse, dq, dk and dv is compared.  The shapes span
several q and k/v tiles, ragged tails (G not a multiple of the tile sizes),
the wrap group of the shifted heads, GQA and MQA, G = 1, G = N (dense
causal), an odd shift, D = 64 and 128, and the fused RoPE prologue.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from grouped_shifted_attention_amd import ops
from gpu_helpers import LSE_MAX_ABS, assert_close, to_bits, to_f64, to_gpu

pytestmark = pytest.mark.gpu

# name, B, N, H, Hkv, D, G, shift, rope
CASES = [
    ("tiny_n256", 1, 256, 4, 4, 64, 64, 32, None),
    ("ragged_g96_gqa_b2", 2, 192, 4, 2, 64, 96, 48, None),
    ("ragged_g200_d128", 1, 600, 2, 2, 128, 200, 100, None),
    ("dense_causal_g_eq_n", 1, 1024, 2, 2, 128, 1024, 0, None),
    ("odd_shift_g250", 1, 1000, 4, 4, 64, 250, 7, None),
    ("g1_self_only", 1, 64, 2, 2, 64, 1, 0, None),
    ("g8_gqa", 1, 64, 4, 2, 128, 8, 4, None),
    ("mqa_no_shift", 1, 384, 4, 1, 128, 128, 0, None),
    ("multi_tile_g512", 1, 2048, 4, 4, 128, 512, 256, None),
    ("gqa8_rope", 1, 512, 16, 2, 128, 256, 128, (10000.0, 8.0)),
    ("rope_d64_b2", 2, 256, 4, 4, 64, 128, 64, (500.0, 2.0)),
    ("ragged_rope_g160", 1, 320, 4, 2, 128, 160, 80, (10000.0, 4.0)),
    ("g2048_large_tiles", 1, 4096, 2, 2, 128, 2048, 1024, None),
    ("ragged_g1100_large_tiles", 1, 2200, 2, 2, 64, 1100, 550, None),
    ("gqa_rope_g1536", 1, 3072, 4, 2, 128, 1536, 768, (10000.0, 8.0)),
    # RoPE scaling variants: position interpolation by 25 out to 100k
    # positions, and the base scaled by 8; dense causal through the
    # eight-wave kernel.
    ("rope_pi25_to_100k", 1, 102400, 2, 2, 128, 4096, 2048, (10000.0, 25.0)),
    ("rope_base8_gqa", 1, 2048, 4, 2, 128, 512, 256, (80000.0, 1.0)),
    ("dense_g4096_large_tiles", 1, 4096, 2, 2, 128, 4096, 0, None),
    # Groups longer than 2048 rows take the eight-wave forward and dQ: a
    # ragged D = 64 group, and grouped-query sharing with RoPE.
    ("ragged_g2200_eight_wave_d64", 1, 4400, 2, 2, 64, 2200, 1100, None),
    ("gqa_rope_g3072_eight_wave", 1, 6144, 4, 2, 128, 3072, 1536, (10000.0, 8.0)),
]
IDS = [c[0] for c in CASES]


def _run(case, seed=0):
    name, B, N, H, Hkv, D, G, sh, rope = case
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=seed)
    q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
    if rope is None:
        out, lse = ops.s2attn_fwd(q, k, v, G, sh)
        dq, dk, dv = ops.s2attn_bwd(q, k, v, out, lse, do, G, sh)
    else:
        out, lse = ops.s2attn_fwd_rope(q, k, v, G, sh, *rope)
        dq, dk, dv = ops.s2attn_bwd_rope(q, k, v, out, lse, do, G, sh, *rope)
    torch.cuda.synchronize()
    x64 = {n: workloads.f64_from_bf16_bits(a) for n, a in x.items()}
    return x64, dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_forward_matches_oracle(case):
    name, B, N, H, Hkv, D, G, sh, rope = case
    x64, got = _run(case)
    ref_o, ref_l = oracle.s2attn_forward(x64["q"], x64["k"], x64["v"], G, sh, rope=rope)
    assert_close("out", to_f64(got["out"]), ref_o)
    assert_close("lse", to_f64(got["lse"]), ref_l, max_abs=LSE_MAX_ABS, half_ulp_rel=0.0)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_backward_matches_oracle(case):
    name, B, N, H, Hkv, D, G, sh, rope = case
    x64, got = _run(case)
    rq, rk, rv = oracle.s2attn_backward(x64["q"], x64["k"], x64["v"], x64["dout"], G, sh, rope=rope)
    assert_close("dq", to_f64(got["dq"]), rq)
    assert_close("dk", to_f64(got["dk"]), rk)
    assert_close("dv", to_f64(got["dv"]), rv)


def test_tiny_workload_against_unrounded_fp32_inputs():
    # The tiny workload is stated with fp32 inputs; the kernel takes bf16.
    # Against the oracle on the unrounded fp32 draws the bar still holds.
    c = workloads.WORKLOADS["tiny_n256"]
    B, N, H, Hkv, D, G, sh = (c[k] for k in ("B", "N", "H", "Hkv", "D", "G", "shift"))
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=0, with_dout=False)
    xf = workloads.make_inputs_f32(B, N, H, Hkv, D, seed=0)
    out, lse = ops.s2attn_fwd(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), G, sh)
    ref_o, ref_l = oracle.s2attn_forward(*(xf[n].astype(np.float64) for n in ("q", "k", "v")), G, sh)
    assert_close("out(fp32 inputs)", to_f64(out), ref_o)
    assert_close("lse(fp32 inputs)", to_f64(lse), ref_l, max_abs=LSE_MAX_ABS, half_ulp_rel=0.0)


def test_llama2_7b_8k_forward_full():
    c = workloads.WORKLOADS["llama2_7b_n8k"]
    B, N, H, Hkv, D, G, sh = (c[k] for k in ("B", "N", "H", "Hkv", "D", "G", "shift"))
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=0, with_dout=False)
    out, lse = ops.s2attn_fwd(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), G, sh)
    x64 = {n: workloads.f64_from_bf16_bits(a) for n, a in x.items()}
    ref_o, ref_l = oracle.s2attn_forward(x64["q"], x64["k"], x64["v"], G, sh)
    assert_close("out", to_f64(out), ref_o)
    assert_close("lse", to_f64(lse), ref_l, max_abs=LSE_MAX_ABS, half_ulp_rel=0.0)


def test_llama2_7b_8k_forward_prescaled_qk():
    # Literal reading of "Q/K pre-scaled by 1/sqrt(D)": the data is scaled;
    # the kernel still applies its 1/sqrt(D) logit scale.
    c = workloads.WORKLOADS["llama2_7b_n8k"]
    B, N, H, Hkv, D, G, sh = (c[k] for k in ("B", "N", "H", "Hkv", "D", "G", "shift"))
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=1, with_dout=False, qk_prescale=D ** -0.5)
    out, lse = ops.s2attn_fwd(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), G, sh)
    x64 = {n: workloads.f64_from_bf16_bits(a) for n, a in x.items()}
    for h, g in ((0, 0), (H - 1, N // G - 1)):
        kvh = oracle.kv_head(h, H, Hkv)
        pos, o, l = oracle.head_unit_forward(x64["q"][0, :, h], x64["k"][0, :, kvh], x64["v"][0, :, kvh],
                                             G, oracle.head_shift(h, H, sh), g)
        assert_close(f"out[h{h},g{g}]", to_f64(out[0, pos, h]), o)
        assert_close(f"lse[h{h},g{g}]", to_f64(lse[0, h, pos]), l, max_abs=LSE_MAX_ABS, half_ulp_rel=0.0)


def test_repeat_calls_are_bitwise_identical():
    case = ("multi_tile_gqa", 1, 1024, 8, 2, 128, 256, 128, None)
    _, a = _run(case, seed=3)
    _, b = _run(case, seed=3)
    for n in ("out", "dq", "dk", "dv"):
        assert np.array_equal(to_bits(a[n]), to_bits(b[n])), n
    assert torch.equal(a["lse"], b["lse"])


def _guarded(shape, dtype, guard=4096):
    # A tensor inside a larger buffer whose margins hold a known pattern.
    n = int(np.prod(shape))
    buf = torch.full((guard + n + guard,), -7.0, dtype=dtype, device="cuda:0")
    return buf, buf[guard:guard + n].view(*shape)


def _margins_intact(buf, n, guard=4096):
    return bool(torch.all(buf[:guard] == -7.0)) and bool(torch.all(buf[guard + n:] == -7.0))


@pytest.mark.parametrize("rope", [None, (10000.0, 8.0)])
def test_outputs_stay_inside_their_buffers(rope):
    B, N, H, Hkv, D, G, sh = 1, 600, 4, 2, 128, 200, 100
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=5)
    q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
    bo, out = _guarded((B, N, H, D), torch.bfloat16)
    bl, lse = _guarded((B, H, N), torch.float32)
    bq, dq = _guarded((B, N, H, D), torch.bfloat16)
    bk, dk = _guarded((B, N, Hkv, D), torch.bfloat16)
    bv, dv = _guarded((B, N, Hkv, D), torch.bfloat16)
    if rope is None:
        ops.s2attn_fwd(q, k, v, G, sh, out=out, lse=lse)
        ops.s2attn_bwd(q, k, v, out, lse, do, G, sh, dq=dq, dk=dk, dv=dv)
    else:
        ops.s2attn_fwd_rope(q, k, v, G, sh, *rope, out=out, lse=lse)
        ops.s2attn_bwd_rope(q, k, v, out, lse, do, G, sh, *rope, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for buf, t in ((bo, out), (bl, lse), (bq, dq), (bk, dk), (bv, dv)):
        assert _margins_intact(buf, t.numel())
    x64 = {n: workloads.f64_from_bf16_bits(a) for n, a in x.items()}
    ref_o, _ = oracle.s2attn_forward(x64["q"], x64["k"], x64["v"], G, sh, rope=rope)
    assert_close("out", to_f64(out), ref_o)


def test_forward_without_lse():
    case = CASES[0]
    _, B, N, H, Hkv, D, G, sh, _ = case
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=0, with_dout=False)
    out, lse = ops.s2attn_fwd(to_gpu(x["q"]), to_gpu(x["k"]), to_gpu(x["v"]), G, sh, with_lse=False)
    assert lse is None
    x64 = {n: workloads.f64_from_bf16_bits(a) for n, a in x.items()}
    ref_o, _ = oracle.s2attn_forward(x64["q"], x64["k"], x64["v"], G, sh)
    assert_close("out", to_f64(out), ref_o)


def test_empty_inputs():
    for B, N in ((0, 256), (1, 0)):
        q = torch.empty((B, N, 4, 64), dtype=torch.bfloat16, device="cuda:0")
        out, lse = ops.s2attn_fwd(q, q.clone(), q.clone(), 64, 32)
        assert out.numel() == 0 and lse.numel() == 0
        dq, dk, dv = ops.s2attn_bwd(q, q.clone(), q.clone(), out, lse, q.clone(), 64, 32)
        assert dq.numel() == 0


def test_invalid_arguments_raise_before_launch():
    q = torch.zeros((1, 256, 4, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(RuntimeError, match="multiple of G"):
        ops.s2attn_fwd(q, q.clone(), q.clone(), 100, 50)
    with pytest.raises(RuntimeError, match="64 or 128"):
        z = torch.zeros((1, 256, 4, 96), dtype=torch.bfloat16, device="cuda:0")
        ops.s2attn_fwd(z, z.clone(), z.clone(), 64, 32)
    with pytest.raises(ValueError):
        ops.s2attn_fwd(q.float(), q, q, 64, 32)


def test_autograd_wrapper_matches_oracle():
    B, N, H, Hkv, D, G = 1, 512, 4, 2, 128, 128
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=7)
    q, k, v, do = (to_gpu(x[n]).requires_grad_(n != "dout") for n in ("q", "k", "v", "dout"))
    out = ops.s2attn(q, k, v, G)  # shift defaults to G // 2
    out.backward(do)
    x64 = {n: workloads.f64_from_bf16_bits(a) for n, a in x.items()}
    ref_o, _ = oracle.s2attn_forward(x64["q"], x64["k"], x64["v"], G, G // 2)
    rq, rk, rv = oracle.s2attn_backward(x64["q"], x64["k"], x64["v"], x64["dout"], G, G // 2)
    assert_close("out", to_f64(out.detach()), ref_o)
    assert_close("dq", to_f64(q.grad), rq)
    assert_close("dk", to_f64(k.grad), rk)
    assert_close("dv", to_f64(v.grad), rv)


def test_backward_stages_equal_the_composite_call():
    B, N, H, Hkv, D, G, sh = 1, 1024, 8, 4, 128, 256, 128
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=11)
    q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
    out, lse = ops.s2attn_fwd(q, k, v, G, sh)
    dq, dk, dv = ops.s2attn_bwd(q, k, v, out, lse, do, G, sh)
    ws = ops.bwd_workspace(q, k)
    ops.s2attn_bwd_preprocess(out, do, lse, ws)
    dk2, dv2 = ops.s2attn_bwd_dkdv(q, k, v, do, G, sh, ws)
    dq2 = ops.s2attn_bwd_dq(q, k, v, do, G, sh, ws)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.array_equal(to_bits(a), to_bits(b))


# Alternate-head shifting through the general entry points: without sharing
# (odd H included, with the four- and the eight-wave kernels), with
# grouped-query sharing and RoPE, and with one k/v head (no head is then
# shifted).
ALT_CASES = [
    ("alt_mha", 1, 512, 4, 4, 64, 128, 64, None),
    ("alt_gqa_rope", 1, 1024, 8, 4, 128, 256, 128, (10000.0, 8.0)),
    ("alt_odd_heads_large_tiles", 1, 4096, 3, 3, 128, 2048, 1024, None),
    ("alt_odd_heads_eight_wave", 1, 5120, 3, 3, 128, 2560, 1280, None),
    ("alt_mqa", 1, 512, 4, 1, 64, 128, 64, None),
]


@pytest.mark.parametrize("case", ALT_CASES, ids=[c[0] for c in ALT_CASES])
def test_alternate_heads_match_oracle(case):
    name, B, N, H, Hkv, D, G, sh, rope = case
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=1)
    q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
    out, lse = ops.s2attn_fwd_ex(q, k, v, G, sh, head_pattern="alternate", rope=rope)
    dq, dk, dv = ops.s2attn_bwd_ex(q, k, v, out, lse, do, G, sh, head_pattern="alternate", rope=rope)
    torch.cuda.synchronize()
    x64 = {n: workloads.f64_from_bf16_bits(a) for n, a in x.items()}
    ref_o, ref_l = oracle.s2attn_forward(x64["q"], x64["k"], x64["v"], G, sh, rope=rope, head_pattern="alternate")
    assert_close("out", to_f64(out), ref_o)
    assert_close("lse", to_f64(lse), ref_l, max_abs=LSE_MAX_ABS, half_ulp_rel=0.0)
    rq, rk, rv = oracle.s2attn_backward(x64["q"], x64["k"], x64["v"], x64["dout"], G, sh, rope=rope,
                                        head_pattern="alternate")
    assert_close("dq", to_f64(dq), rq)
    assert_close("dk", to_f64(dk), rk)
    assert_close("dv", to_f64(dv), rv)


def test_general_entry_points_match_the_specific_ones():
    # Second-half pattern through s2attn_fwd_ex / s2attn_bwd_ex equals
    # s2attn_fwd / s2attn_bwd bit for bit (same kernels, same arguments).
    B, N, H, Hkv, D, G, sh = 1, 512, 4, 2, 128, 128, 64
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=2)
    q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
    out, lse = ops.s2attn_fwd(q, k, v, G, sh)
    dq, dk, dv = ops.s2attn_bwd(q, k, v, out, lse, do, G, sh)
    out2, lse2 = ops.s2attn_fwd_ex(q, k, v, G, sh)
    dq2, dk2, dv2 = ops.s2attn_bwd_ex(q, k, v, out2, lse2, do, G, sh)
    for a, b in ((out, out2), (dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse, lse2)
