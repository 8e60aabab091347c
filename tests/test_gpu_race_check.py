"""Race check: the race-check build (S2A_DEBUG_BARRIERS: every LDS hand-over
drains all outstanding memory operations and meets a full barrier) must give
the normal build's results bit for bit.  A hand-over that relies on a missing
wait or barrier shows up as a difference, on a ragged shape, a grouped-query
shape with RoPE, the LLaMA2-7B 32k workload and a LoRA projection."""
import pytest
import torch

import workloads
from grouped_shifted_attention_amd import _lib, ops
from grouped_shifted_attention_amd.build import DEBUG_LIB_PATH
from gpu_helpers import to_gpu

pytestmark = pytest.mark.gpu

# name, B, N, H, Hkv, D, G, shift, rope
CASES = [
    ("ragged_g200_gqa", 2, 600, 4, 2, 128, 200, 100, None),
    ("gqa8_rope", 1, 512, 16, 2, 128, 256, 128, (10000.0, 8.0)),
    ("ragged_g1100_d64", 1, 2200, 2, 2, 64, 1100, 550, None),
    ("llama2_7b_n32k", 1, 32768, 32, 32, 128, 8192, 4096, None),
]


def _attention(case):
    name, B, N, H, Hkv, D, G, sh, rope = case
    x = workloads.make_inputs(B, N, H, Hkv, D, seed=3)
    q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
    if rope is None:
        out, lse = ops.s2attn_fwd(q, k, v, G, sh)
        grads = ops.s2attn_bwd(q, k, v, out, lse, do, G, sh)
    else:
        out, lse = ops.s2attn_fwd_rope(q, k, v, G, sh, *rope)
        grads = ops.s2attn_bwd_rope(q, k, v, out, lse, do, G, sh, *rope)
    torch.cuda.synchronize()
    return (out, lse) + tuple(grads)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_race_check_build_matches_bit_for_bit(case):
    normal = _attention(case)
    with _lib.using(_lib.load(DEBUG_LIB_PATH)):
        checked = _attention(case)
    for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), normal, checked):
        assert torch.equal(a.view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                           b.view(torch.int32 if b.dtype == torch.float32 else torch.int16)), name


def test_race_check_build_matches_lora_projections():
    M, d_in, wq, wkv, r = 600, 256, 512, 256, 64
    lx = workloads.make_lora_inputs(M, d_in, (wq, wkv, wkv), r, seed=4, with_dy=True)
    g = to_gpu

    x, wt = g(lx["x"]), [g(w) for w in lx["wt"]]
    at, bt, dys = [g(a) for a in lx["at"]], [g(b) for b in lx["bt"]], [g(d) for d in lx["dy"]]

    def run():
        q, k, v, ws = ops.s2attn_lora_qkv_fwd(x, wt, at, bt, 1.0)
        t = ws[: M * 3 * r * 2].view(torch.bfloat16).view(M, 3 * r)
        dx, dat, dbt = ops.s2attn_lora_qkv_bwd(x, wt, at, bt, 1.0, t, dys)
        torch.cuda.synchronize()
        return [q, k, v, t.clone(), dx] + list(dat) + list(dbt)

    normal = run()
    with _lib.using(_lib.load(DEBUG_LIB_PATH)):
        checked = run()
    assert len(normal) == len(checked)
    for i, (a, b) in enumerate(zip(normal, checked)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), i
