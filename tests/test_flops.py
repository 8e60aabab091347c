"""The benchmark's FLOP accounting, pinned to the numbers the pages print."""
import json
import os

from grouped_shifted_attention_amd import flops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "flop_demo.json")


def test_guide_flop_demo():
    g = json.load(open(GOLDEN))
    L, dm, G = g["seq_len"], g["d_model"], g["group_size"]
    # The page counts L*G*d_model "ops" (one multiply-add per pair per
    # channel over the causal half of QK^T and PV); FLOPs are twice that.
    for H in (8, 16):
        D = dm // H
        assert flops.s2attn_fwd_flops(1, H, L, G, D) == 2 * g["s2_ops"]
        assert flops.s2attn_fwd_flops(1, H, L, L, D) == 2 * g["dense_ops"]
    saving = 100.0 * (1 - flops.s2attn_fwd_flops(1, 8, L, G, 128) / flops.s2attn_fwd_flops(1, 8, L, L, 128))
    assert round(saving, 1) == g["savings_percent"]


def test_abstract_cost_ratio_and_group_fold():
    g = json.load(open(GOLDEN))
    long_, short = g["abstract_long"], g["abstract_short"]
    dense = lambda n: flops.s2attn_fwd_flops(1, 32, n, n, 128)
    assert dense(long_) // dense(short) == g["abstract_cost_ratio"]
    N = 32768
    assert flops.s2attn_fwd_flops(1, 32, N, N, 128) // flops.s2attn_fwd_flops(1, 32, N, N // 4, 128) \
        == g["aimech_fold_at_quarter"]


def test_backward_is_two_and_a_half_forward():
    assert flops.s2attn_bwd_flops(1, 32, 32768, 8192, 128) * 2 == 5 * flops.s2attn_fwd_flops(1, 32, 32768, 8192, 128)


def test_algorithmic_bytes():
    # LLaMA2-7B at 32k: q, k, v, out (bf16) + lse (fp32)
    assert flops.fwd_algorithmic_bytes(1, 32768, 32, 32, 128) == 1_077_936_128
    assert flops.bwd_algorithmic_bytes(1, 32768, 32, 32, 128) == 2_151_677_952
