"""The entry point that allocates nothing, s2attn_bwd_noalloc, against
s2attn_bwd (same kernels, caller workspace) on two calls in a row, the second
with a smaller input: the outputs must agree bit for bit (and so meet the
parity bar against the oracle that s2attn_bwd meets)."""
import pytest
import torch

import workloads
from grouped_shifted_attention_amd import ops
from gpu_helpers import to_gpu

pytestmark = pytest.mark.gpu

# B, N, H, Hkv, D, G, shift: GQA across several q and k/v tiles, then a
# smaller MHA shape with a ragged group (fewer statistics rows than the first
# call left in the scratch).
SHAPES = [(1, 4096, 8, 4, 128, 2048, 1024), (2, 600, 4, 4, 64, 200, 100)]


def test_noalloc_backward_equals_workspace_backward_twice():
    for B, N, H, Hkv, D, G, sh in SHAPES:
        print(f"  noalloc case B{B} N{N} H{H} Hkv{Hkv} D{D} G{G} shift{sh}", flush=True)
        x = workloads.make_inputs(B, N, H, Hkv, D, seed=B + N)
        q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
        out, lse = ops.s2attn_fwd(q, k, v, G, sh)
        ref = ops.s2attn_bwd(q, k, v, out, lse, do, G, sh)
        got = ops.s2attn_bwd_noalloc(q, k, v, out, lse, do, G, sh)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
