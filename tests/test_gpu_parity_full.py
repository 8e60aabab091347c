"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.

The oracle computes sampled units (batch, head, group) one by one: the first
and last head of each half (H/2 - 1 and H/2 are the last unshifted and the
first shifted head) in the first group and in the last group, which for the
shifted heads is the wrap group.  Under grouped-query sharing the k/v
gradients are compared per (k/v head, group) with all the q heads that read
that k/v head.  Groups are independent, so a sampled unit's rows are
compared exactly with the oracle's.
The whole gradient tensors are additionally checked against invariants that
need no oracle: per (k/v head, group), the key gradients of the rotated keys
sum to zero (softmax rows of dS sum to zero) and the value gradients sum to
the summed output gradients of the q heads that read them (rows of P sum to
one).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from grouped_shifted_attention_amd import ops
from gpu_helpers import LSE_MAX_ABS, assert_close, to_f64, to_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


class Run:
    """Inputs (bit arrays on the host, tensors on the GPU) and the outputs of
    one forward + backward at a workload's full size."""

    def __init__(self, name, seed=0):
        c = workloads.WORKLOADS[name]
        self.name = name
        self.B, self.N, self.H, self.Hkv, self.D, self.G, self.sh = (
            c[k] for k in ("B", "N", "H", "Hkv", "D", "G", "shift"))
        self.rope = c["rope"]
        self.pattern = c.get("head_pattern", "second_half")
        print(f"  generating {name}", flush=True)
        self.x = workloads.make_inputs(self.B, self.N, self.H, self.Hkv, self.D, seed=seed)
        q, k, v, do = (to_gpu(self.x[n]) for n in ("q", "k", "v", "dout"))
        print(f"  running {name} on the GPU", flush=True)
        if self.pattern != "second_half":
            self.out, self.lse = ops.s2attn_fwd_ex(q, k, v, self.G, self.sh, head_pattern=self.pattern,
                                                   rope=self.rope)
            self.dq, self.dk, self.dv = ops.s2attn_bwd_ex(q, k, v, self.out, self.lse, do, self.G, self.sh,
                                                          head_pattern=self.pattern, rope=self.rope)
        elif self.rope is None:
            self.out, self.lse = ops.s2attn_fwd(q, k, v, self.G, self.sh)
            self.dq, self.dk, self.dv = ops.s2attn_bwd(q, k, v, self.out, self.lse, do, self.G, self.sh)
        else:
            self.out, self.lse = ops.s2attn_fwd_rope(q, k, v, self.G, self.sh, *self.rope)
            self.dq, self.dk, self.dv = ops.s2attn_bwd_rope(q, k, v, self.out, self.lse, do, self.G, self.sh,
                                                            *self.rope)
        torch.cuda.synchronize()
        self.do = do
        self.NG = self.N // self.G

    def shift_of(self, h):
        return oracle.head_shift(h, self.H, self.sh, self.pattern, self.Hkv)

    def head(self, name, h):
        return workloads.f64_from_bf16_bits(self.x[name][0, :, h, :])

    def check_forward_unit(self, h, g):
        kvh = oracle.kv_head(h, self.H, self.Hkv)
        pos, o, l = oracle.head_unit_forward(self.head("q", h), self.head("k", kvh), self.head("v", kvh),
                                             self.G, self.shift_of(h), g, rope=self.rope)
        idx = torch.from_numpy(pos).cuda()
        assert_close(f"out[h{h},g{g}]", to_f64(self.out[0, :, h][idx]), o)
        assert_close(f"lse[h{h},g{g}]", to_f64(self.lse[0, h][idx]), l, max_abs=LSE_MAX_ABS, half_ulp_rel=0.0)

    def check_backward_kv_group(self, kvh, g, check_dq_heads=None):
        """dk, dv of k/v head kvh in group g summed over its q heads; dq of
        the q heads in check_dq_heads (all of them by default)."""
        r = self.H // self.Hkv
        heads = list(range(kvh * r, (kvh + 1) * r))
        dk = dv = None
        for h in heads:
            pos, uq, uk, uv = oracle.head_unit_backward(
                self.head("q", h), self.head("k", kvh), self.head("v", kvh), self.head("dout", h),
                self.G, self.shift_of(h), g, rope=self.rope)
            dk = uk if dk is None else dk + uk
            dv = uv if dv is None else dv + uv
            if check_dq_heads is None or h in check_dq_heads:
                idx = torch.from_numpy(pos).cuda()
                assert_close(f"dq[h{h},g{g}]", to_f64(self.dq[0, :, h][idx]), uq)
        idx = torch.from_numpy(pos).cuda()
        assert_close(f"dk[kv{kvh},g{g}]", to_f64(self.dk[0, :, kvh][idx]), dk)
        assert_close(f"dv[kv{kvh},g{g}]", to_f64(self.dv[0, :, kvh][idx]), dv)

    def check_gradient_invariants(self, tol=2e-3):
        r = self.H // self.Hkv
        worst_k = worst_v = 0.0
        for kvh in range(self.Hkv):
            sh = self.shift_of(kvh * r)
            dk = self.dk[0, :, kvh].float()
            if self.rope is not None:
                # Gradient w.r.t. the rotated keys: rotate the returned one.
                dk64 = oracle.rope_rotate(to_f64(self.dk[0, :, kvh]), np.arange(self.N), *self.rope)
                dk = torch.from_numpy(dk64).cuda()
            dk = torch.roll(dk, -sh, dims=0).view(self.NG, self.G, self.D)
            dv = torch.roll(self.dv[0, :, kvh].float(), -sh, dims=0).view(self.NG, self.G, self.D)
            do = torch.roll(self.do[0, :, kvh * r:(kvh + 1) * r].float().sum(1), -sh, dims=0)
            do = do.view(self.NG, self.G, self.D)
            ratio_k = (dk.sum(1).norm(dim=1) / dk.norm(dim=2).sum(1)).max().item()
            ratio_v = ((dv.sum(1) - do.sum(1)).norm(dim=1) / do.norm(dim=2).sum(1)).max().item()
            worst_k, worst_v = max(worst_k, ratio_k), max(worst_v, ratio_v)
        print(f"  invariants: |sum dk|/sum|dk| <= {worst_k:.2e}, |sum dv - sum do|/sum|do| <= {worst_v:.2e}",
              flush=True)
        assert worst_k <= tol and worst_v <= tol
        for t in (self.out, self.dq, self.dk, self.dv):
            assert bool(torch.isfinite(t).all())


_runs = {}


def run_of(name):
    if name not in _runs:
        _runs.clear()  # keep one workload's tensors on the GPU at a time
        torch.cuda.empty_cache()
        _runs[name] = Run(name)
    return _runs[name]


def sample_units(heads, groups):
    """Units (head, group) of a workload: the first and last head of each
    half (H/2 - 1 and H/2 border the shift) in the first and last group."""
    return [(h, g) for h in (0, heads // 2 - 1, heads // 2, heads - 1) for g in (0, groups - 1)]


# ---------------------------------------------------------------- 7B, 32k

@pytest.mark.parametrize("h,g", sample_units(32, 4))
def test_llama2_7b_32k_forward_units(h, g):
    run_of("llama2_7b_n32k").check_forward_unit(h, g)


@pytest.mark.parametrize("kvh,g", sample_units(32, 4))
def test_llama2_7b_32k_backward_units(kvh, g):
    run_of("llama2_7b_n32k").check_backward_kv_group(kvh, g)


def test_llama2_7b_32k_gradient_invariants():
    run_of("llama2_7b_n32k").check_gradient_invariants()


def test_llama2_7b_32k_deterministic():
    r = run_of("llama2_7b_n32k")
    q, k, v = (to_gpu(r.x[n]) for n in ("q", "k", "v"))
    out, lse = ops.s2attn_fwd(q, k, v, r.G, r.sh)
    dq, dk, dv = ops.s2attn_bwd(q, k, v, out, lse, r.do, r.G, r.sh)
    for a, b in ((out, r.out), (dq, r.dq), (dk, r.dk), (dv, r.dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse, r.lse)


# --------------------------------------------------- 70B-style GQA + RoPE

@pytest.mark.parametrize("h,g", sample_units(64, 4))
def test_gqa_rope_32k_forward_units(h, g):
    run_of("llama2_70b_gqa_n32k_rope").check_forward_unit(h, g)


# k/v heads 3 and 4 are the last unshifted and the first shifted one; each
# is compared with all 8 of its q heads.
@pytest.mark.parametrize("kvh,g", sample_units(8, 4))
def test_gqa_rope_32k_backward_units(kvh, g):
    run_of("llama2_70b_gqa_n32k_rope").check_backward_kv_group(kvh, g)


def test_gqa_rope_32k_gradient_invariants():
    run_of("llama2_70b_gqa_n32k_rope").check_gradient_invariants()


# ---------------------------------------------------------------- 7B, 100k

@pytest.mark.parametrize("h,g", sample_units(32, 4))
def test_llama2_7b_100k_forward_units(h, g):
    run_of("llama2_7b_n100k").check_forward_unit(h, g)


@pytest.mark.parametrize("kvh,g", sample_units(32, 4))
def test_llama2_7b_100k_backward_units(kvh, g):
    run_of("llama2_7b_n100k").check_backward_kv_group(kvh, g)


def test_llama2_7b_100k_gradient_invariants():
    run_of("llama2_7b_n100k").check_gradient_invariants()


# ------------------------------------------- dense causal (inference mode)

@pytest.mark.parametrize("h", [0, 31])
def test_dense_32k_forward_units(h):
    run_of("llama2_7b_dense_n32k").check_forward_unit(h, 0)


def test_dense_32k_backward_unit():
    run_of("llama2_7b_dense_n32k").check_backward_kv_group(16, 0)


def test_dense_32k_gradient_invariants():
    run_of("llama2_7b_dense_n32k").check_gradient_invariants()


# ------------------------------- RoPE scaling: PI by 25 at 100k, base x 8

@pytest.mark.parametrize("h,g", [(0, 0), (31, 3)])
def test_rope_pi25_100k_forward_units(h, g):
    run_of("llama2_7b_n100k_rope_pi25").check_forward_unit(h, g)


def test_rope_pi25_100k_backward_unit():
    run_of("llama2_7b_n100k_rope_pi25").check_backward_kv_group(31, 3)


def test_rope_pi25_100k_gradient_invariants():
    run_of("llama2_7b_n100k_rope_pi25").check_gradient_invariants()


@pytest.mark.parametrize("h,g", [(3, 1), (20, 3)])
def test_rope_base8_32k_forward_units(h, g):
    run_of("llama2_7b_n32k_rope_base8").check_forward_unit(h, g)


def test_rope_base8_32k_backward_unit():
    run_of("llama2_7b_n32k_rope_base8").check_backward_kv_group(20, 3)


# ------------------------------------------------ alternate heads shifted

@pytest.mark.parametrize("h,g", [(0, 3), (1, 0), (30, 1), (31, 3)])
def test_alternate_32k_forward_units(h, g):
    run_of("llama2_7b_n32k_alternate").check_forward_unit(h, g)


@pytest.mark.parametrize("kvh,g", [(1, 3), (30, 0)])
def test_alternate_32k_backward_units(kvh, g):
    run_of("llama2_7b_n32k_alternate").check_backward_kv_group(kvh, g)


def test_alternate_32k_gradient_invariants():
    run_of("llama2_7b_n32k_alternate").check_gradient_invariants()
