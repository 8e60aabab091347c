"""The seeded input generator: bf16 rounding checked against torch's own
float32 -> bfloat16 conversion (round to nearest even), exact widening, and
reproducible draws."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(200_000).astype(np.float32)
    x[:8] = [1.0, -2.5, 3.0e38, -3.0e38, 1e-40, 0.0, 1.00390625, 1.01171875]  # incl. ties
    got = workloads.bf16_bits_from_f32(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite values only
    w = workloads.f64_from_bf16_bits(bits)
    back = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(back, bits)


def test_non_finite_input_is_rejected():
    with pytest.raises(ValueError):
        workloads.bf16_bits_from_f32(np.array([np.inf], np.float32))


def test_draws_are_seeded_and_ordered():
    a = workloads.make_inputs(1, 16, 4, 2, 8, seed=3)
    b = workloads.make_inputs(1, 16, 4, 2, 8, seed=3)
    for n in ("q", "k", "v", "dout"):
        assert np.array_equal(a[n], b[n])
    assert a["q"].shape == (1, 16, 4, 8) and a["k"].shape == (1, 16, 2, 8)
    f = workloads.make_inputs_f32(1, 16, 4, 2, 8, seed=3)
    assert np.array_equal(workloads.bf16_bits_from_f32(f["q"]), a["q"])
    c = workloads.make_inputs(1, 16, 4, 2, 8, seed=4)
    assert not np.array_equal(a["q"], c["q"])


def test_workload_shapes_are_consistent():
    for name, c in workloads.WORKLOADS.items():
        assert c["N"] % c["G"] == 0, name
        assert c["H"] % c["Hkv"] == 0 and c["H"] % 2 == 0 and c["Hkv"] % 2 == 0, name
        if c["G"] == c["N"]:
            assert c["shift"] == 0, name  # dense causal: one group, nothing to shift
        else:
            assert c["shift"] == c["G"] // 2, name
            assert c["G"] * 4 == c["N"], name  # G = N/4 for every S2-Attn shape
    assert workloads.BENCH_WORKLOAD in workloads.WORKLOADS
