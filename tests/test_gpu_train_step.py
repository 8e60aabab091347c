"""The LongLoRA attention training step end to end, against the chained oracles.

x -> LoRA-adapted q/k/v projections -> S2-Attn (optionally with RoPE and
position interpolation) -> loss <out, dout> -> gradients of x and of the
adapters.  The GPU side goes through the autograd wrappers (every product in
the library's kernels, bf16 between stages); the reference chains the fp64
oracles (oracle.lora_qkv_forward, oracle.s2attn_forward / s2attn_backward,
oracle.lora_qkv_backward) with no rounding between stages.  Bar: rel-L2
<= 1e-2 on the attention output and on every gradient (the per-stage bar; the
bf16 hand-overs between stages add a few 1e-3 at most).
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

# name, N, H, Hkv, D, G, shift, r, scale, rope
CASES = [
    ("mha_g128", 512, 4, 4, 64, 128, 64, 16, 1.0, None),
    ("gqa_rope_pi4", 512, 4, 2, 64, 128, 64, 16, 0.5, (10000.0, 4.0)),
    ("d128_g256", 1024, 2, 2, 128, 256, 128, 64, 1.0, None),
]


def _rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_lora_s2attn_training_step(case):
    name, N, H, Hkv, D, G, shift, r, scale, rope = case
    d_in, wq, wkv = H * D, H * D, Hkv * D
    d = workloads.make_lora_inputs(N, d_in, (wq, wkv, wkv), r, seed=31)
    dout_bits = workloads.make_inputs(1, N, H, Hkv, D, seed=32)["dout"]

    # GPU: autograd through the library.
    x = to_gpu(d["x"]).requires_grad_(True)
    wt = [to_gpu(w) for w in d["wt"]]
    at = [to_gpu(a).requires_grad_(True) for a in d["at"]]
    bt = [to_gpu(b).requires_grad_(True) for b in d["bt"]]
    q, k, v = ops.lora_qkv(x, wt, at, bt, scale)
    out = ops.s2attn(q.view(1, N, H, D), k.view(1, N, Hkv, D), v.view(1, N, Hkv, D), G, shift, rope)
    out.backward(to_gpu(dout_bits))
    torch.cuda.synchronize()

    # Reference: the fp64 oracles chained.
    xf = f64_from_bf16_bits(d["x"])
    Ws = [f64_from_bf16_bits(w).T for w in d["wt"]]
    ads = [(f64_from_bf16_bits(a).T, f64_from_bf16_bits(b).T) for a, b in zip(d["at"], d["bt"])]
    yq, yk, yv = oracle.lora_qkv_forward(xf, Ws, ads, scale)
    q4, k4, v4 = yq.reshape(1, N, H, D), yk.reshape(1, N, Hkv, D), yv.reshape(1, N, Hkv, D)
    ref_out, _ = oracle.s2attn_forward(q4, k4, v4, G, shift, rope=rope)
    dout = f64_from_bf16_bits(dout_bits)
    dq, dk, dv = oracle.s2attn_backward(q4, k4, v4, dout, G, shift, rope=rope)
    ref_dx, grads = oracle.lora_qkv_backward(xf, Ws, ads, scale,
                                             [dq.reshape(N, wq), dk.reshape(N, wkv), dv.reshape(N, wkv)])

    checks = [("out", to_f64(out.detach()), ref_out), ("dx", to_f64(x.grad), ref_dx)]
    for p in range(3):
        checks.append((f"dA_{'qkv'[p]}^T", to_f64(at[p].grad), grads[p][0].T))
        checks.append((f"dB_{'qkv'[p]}^T", to_f64(bt[p].grad), grads[p][1].T))
    for nm, got, ref in checks:
        rel = _rel(got, ref)
        print(f"  {nm}: rel-L2 {rel:.2e}", flush=True)
        assert rel <= 1e-2, f"{nm}: rel-L2 {rel:.3e}"
    for w in wt:
        assert w.grad is None  # frozen
