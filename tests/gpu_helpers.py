"""Helpers shared by the GPU parity tests (marshalling and error metrics)."""
import json
import os

import numpy as np
import torch

from workloads import f64_from_bf16_bits

# Parity bar for bf16 outputs and gradients with fp32 accumulation:
#   rel-L2  = ||got - ref|| / ||ref||                          <= 1e-2
#   max-abs = max |got - ref| beyond the output's own rounding <= 2e-2
# The outputs are bf16, whose half-ulp is |ref| * 2^-8; above magnitude 4
# that rounding alone exceeds 2e-2 (k/v gradients summed over grouped-query
# heads reach 4..16), so each element may additionally differ by its own
# half-ulp.  The same bar holds for every tensor, grouped-query k/v
# gradients included.
MAX_ABS = 2e-2
REL_L2 = 1e-2
BF16_HALF_ULP_REL = 2.0 ** -8


# The log-sum-exp is fp32 (no output rounding); its error comes from the bf16
# logits' rounding, a few 1e-3 at these magnitudes; same absolute bar.
LSE_MAX_ABS = 2e-2


def to_gpu(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit array -> contiguous bf16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda:0").view(torch.bfloat16)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return f64_from_bf16_bits(to_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray, half_ulp_rel=BF16_HALF_ULP_REL):
    """(max-abs beyond rounding, rel-L2, plain max-abs, |ref| at the worst element)."""
    d = np.abs(got - ref)
    if d.size == 0:
        return 0.0, 0.0, 0.0, 0.0
    excess = d - half_ulp_rel * np.abs(ref)
    i = int(np.argmax(excess))
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got - ref))
    return float(excess.flat[i]), rel, float(d.max()), float(abs(ref.flat[i]))


# When S2A_PARITY_LOG names a file, every comparison appends one JSON line
# to it (test, tensor, errors, bars), so a run's margins survive pytest's
# output capture.
PARITY_LOG = os.environ.get("S2A_PARITY_LOG")


def log_margin(name, **fields):
    if not PARITY_LOG:
        return
    rec = dict(test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], tensor=name, **fields)
    with open(PARITY_LOG, "a") as f:
        f.write(json.dumps(rec) + "\n")


def assert_close(name, got, ref, max_abs=MAX_ABS, rel_l2=REL_L2, half_ulp_rel=BF16_HALF_ULP_REL):
    m, r, plain, at = errors(got, ref, half_ulp_rel)
    print(f"  {name}: max_abs_beyond_rounding={m:.3e} (|ref| there {at:.3g}) plain_max_abs={plain:.3e} "
          f"rel_l2={r:.3e}", flush=True)
    log_margin(name, beyond_rounding=m, plain_max_abs=plain, rel_l2=r, ref_at_worst=at, bar_max_abs=max_abs,
               bar_rel_l2=rel_l2, rounding_allowance=half_ulp_rel, n=int(np.size(ref)))
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert m <= max_abs, f"{name}: max_abs beyond rounding {m:.3e} > {max_abs}"
    assert r <= rel_l2, f"{name}: rel_l2 {r:.3e} > {rel_l2}"
