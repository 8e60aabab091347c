#!/usr/bin/env python3
"""S2-Attn forward + backward throughput on one MI355X.

One step is the whole hot path over one batch of synthetic input: the forward
kernel, then the backward's three kernels (Delta preprocess, dK/dV, dQ), on
the LLaMA2-7B attention shape at 32k context (B 1, N 32768, H 32, D 128,
G 8192, shift 4096) unless --workload says otherwise.  Inputs are seeded
N(0, 1) draws rounded to bf16 and stay resident in HBM.

Throughput counts effective causal FLOPs: 2*B*H*N*G*D forward plus 2.5x that
backward, over the wall time of K steps bracketed by device synchronisation.
Each kernel is also bracketed by HIP events recorded on the stream the
kernels are launched on; their average durations give the roofline of the
dominant kernel.

Prints ONE JSON line.  Options:
  --gpus N        only 1 is supported (the path is single-GPU)
  --steps K       timed steps (default 20)
  --warmup W      untimed steps first (default 5)
  --workload W    a key of workloads.WORKLOADS (with RoPE or alternate-head
                  shifting: the general entry points are timed as two calls,
                  forward and backward), or of workloads.LORA_WORKLOADS: the
                  LoRA q/k/v projections ahead of the attention, one call
                  per step, with the library GEMM timed beside for context
  --no-cpu-baseline   skip timing the fp64 oracle on a sample
  --calib-copy-mib M  also run one plain device copy of M MiB (for counter calibration)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
METRIC = "S2-Attn fwd+bwd TFLOP/s and % bf16 MFMA peak, LLaMA2-7B shape N=32k G=8k"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = ["fwd.hip", "bwd.hip", "bwd_delta.hip", "staging.hpp", "device_common.hpp", "kernels.hpp"]


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "grouped_shifted_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def cpu_baseline(cfg, x_bits, budget_s=20.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole (batch, head, group) units, forward + backward, until the
    budget is used; report effective TFLOP/s under the same FLOP convention."""
    import numpy as np

    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:  # threadpoolctl absent
        blas = []
    B, N, H, Hkv, D, G, sh = (cfg[k] for k in ("B", "N", "H", "Hkv", "D", "G", "shift"))
    units = [(h, g) for g in (0, N // G - 1) for h in (0, H // 2, H - 1, H // 2 - 1)]
    done = 0
    t0 = time.perf_counter()
    for h, g in units:
        kvh = oracle.kv_head(h, H, Hkv)
        f64 = lambda name, hh: workloads.f64_from_bf16_bits(x_bits[name][0, :, hh, :])
        qh, kh, vh, doh = f64("q", h), f64("k", kvh), f64("v", kvh), f64("dout", h)
        shh = oracle.head_shift(h, H, sh, cfg.get("head_pattern", "second_half"), Hkv)
        oracle.head_unit_forward(qh, kh, vh, G, shh, g, rope=cfg["rope"])
        oracle.head_unit_backward(qh, kh, vh, doh, G, shh, g, rope=cfg["rope"])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = done * 7 * G * G * D  # per unit: 2 G^2 D forward + 5 G^2 D backward
    threads = max([n for _, n in blas if n] or [1])
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {B * H * (N // G)} (batch, head, group) units of {cfg['name']}, forward + "
                  f"backward in float64 NumPy, {dt:.1f} s; every unit does identical work, so the rate "
                  f"is the whole workload's",
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas": blas,
        "seconds": dt,
    }


def calib_copy(args, dev):
    """One plain device copy of --calib-copy-mib MiB (counter calibration)."""
    import torch
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


LORA_METRIC = "LoRA q/k/v projection fwd+bwd TFLOP/s and % bf16 MFMA peak"


def lora_flops(M, d_in, widths, r):
    """MFMA work of one projection call: the frozen products, x A and (x A) B."""
    wsum = sum(widths)
    return 2.0 * M * d_in * wsum + 2.0 * M * d_in * 3 * r + 2.0 * M * r * wsum


def lora_bwd_flops(M, d_in, widths, r):
    """MFMA work of the backward: dy B^T, dx (frozen and low-rank parts), dA, dB."""
    wsum = sum(widths)
    return 2.0 * M * r * wsum + 2.0 * M * d_in * (wsum + 3 * r) + 2.0 * M * 3 * r * d_in + 2.0 * M * wsum * r


def lora_cpu_baseline(cfg, d, dy_bits, budget_s):
    """The fp64 oracle, forward and backward, on a bounded sample of token
    rows of the same inputs (the backward's token reductions are linear in
    the rows, so a row block does its share of every product)."""
    import numpy as np

    import oracle
    from workloads import f64_from_bf16_bits
    M, d_in, widths, r, s = cfg["M"], cfg["d_in"], cfg["widths"], cfg["r"], cfg["scale"]
    Ws = [f64_from_bf16_bits(w).T for w in d["wt"]]
    ads = [(f64_from_bf16_bits(a).T, f64_from_bf16_bits(b).T) for a, b in zip(d["at"], d["bt"])]
    rows, done = 256, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < M:
        x = f64_from_bf16_bits(d["x"][done:done + rows])
        oracle.lora_qkv_forward(x, Ws, ads, s)
        oracle.lora_qkv_backward(x, Ws, ads, s, [f64_from_bf16_bits(g[done:done + rows]) for g in dy_bits])
        done += x.shape[0]
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:
        blas = []
    return {
        "value": (lora_flops(done, d_in, widths, r) + lora_bwd_flops(done, d_in, widths, r)) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": max([n for _, n in blas if n] or [1]),
        "kind": "oracle",
        "sample": f"the first {done} of {M} token rows of {cfg['name']} (all three projections, forward + backward), float64 "
                  f"NumPy, {dt:.1f} s; rows do identical work, so the rate is the whole workload's",
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas": blas,
        "seconds": dt,
    }


def bench_lora(args, name):
    import numpy as np
    import torch
    import torch.nn.functional as F

    import workloads
    from grouped_shifted_attention_amd import ops
    cfg = dict(workloads.LORA_WORKLOADS[name], name=name)
    M, d_in, widths, r, s = cfg["M"], cfg["d_in"], cfg["widths"], cfg["r"], cfg["scale"]
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = workloads.make_lora_inputs(M, d_in, widths, r, seed=0)
    to_gpu = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    x = to_gpu(d["x"])
    wt = [to_gpu(w) for w in d["wt"]]
    at = [to_gpu(a) for a in d["at"]]
    bt = [to_gpu(b) for b in d["bt"]]
    dy_bits = workloads.make_lora_inputs(M, d_in, widths, r, seed=1, with_dy=True)["dy"]
    dys = [to_gpu(g) for g in dy_bits]
    outs = tuple(torch.empty(M, w, dtype=torch.bfloat16, device=dev) for w in widths)
    ws = ops.lora_qkv_workspace(M, r, dev)
    t = ws[: M * 3 * r * 2].view(torch.bfloat16).view(M, 3 * r)
    grads = (torch.empty(M, d_in, dtype=torch.bfloat16, device=dev),
             [torch.empty(r, d_in, dtype=torch.bfloat16, device=dev) for _ in range(3)],
             [torch.empty(w, r, dtype=torch.bfloat16, device=dev) for w in widths])
    wsb = ops.lora_qkv_bwd_workspace(M, d_in, widths[0], widths[1], r, dev)
    calib_copy(args, dev)
    stream = torch.cuda.current_stream(dev)

    # One step: the projections forward, then their backward for a fixed
    # upstream gradient (the training step of the prologue).
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ops.s2attn_lora_qkv_fwd(x, wt, at, bt, s, out=outs, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        ops.s2attn_lora_qkv_bwd(x, wt, at, bt, s, t, dys, out=grads, workspace=wsb)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ffl, bfl = lora_flops(M, d_in, widths, r), lora_bwd_flops(M, d_in, widths, r)
    value = (ffl + bfl) / (ms_step * 1e-3) / 1e12
    kernel_flops = {"lora_fwd_call": ffl, "lora_bwd_call": bfl}
    kernel_ms = {"lora_fwd_call": fwd_ms, "lora_bwd_call": bwd_ms}
    dominant = max(kernel_ms, key=kernel_ms.get)
    achieved = kernel_flops[dominant] / (kernel_ms[dominant] * 1e-3) / 1e12

    # Context: the library GEMM (hipBLASLt through torch) for the frozen part
    # alone, all three weights concatenated into one [sum(widths), d_in].
    wcat = torch.cat(wt, 0).contiguous()
    for _ in range(3):
        F.linear(x, wcat)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        F.linear(x, wcat)
    e1.record(stream)
    torch.cuda.synchronize()
    lib_ms = e0.elapsed_time(e1) / 10
    lib_tf = 2.0 * M * d_in * sum(widths) / (lib_ms * 1e-3) / 1e12
    alg_bytes = 2.0 * (M * d_in + sum(widths) * d_in + M * sum(widths) + 3 * r * d_in + sum(widths) * r
                       + 2 * M * 3 * r)
    line = {
        "metric": LORA_METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "M": M, "d_in": d_in, "widths": list(widths), "r": r, "scale": s,
                   "parallelism": "single-gpu", "operands": args.operands},
        "pct_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd_tflops": ffl / (fwd_ms * 1e-3) / 1e12,
        "bwd_tflops": bfl / (bwd_ms * 1e-3) / 1e12,
        "kernel_ms": kernel_ms,
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": None, "avg_launch_ms": kernel_ms[dominant]},
        "hbm_gbs_algorithmic": {"fwd_call": alg_bytes / (fwd_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS},
        "library_frozen_gemm": {"what": "torch F.linear (hipBLASLt) of x by the three frozen weights "
                                        "concatenated, no adapter", "ms": lib_ms, "tflops": lib_tf},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = lora_cpu_baseline(cfg, d, dy_bits, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0)
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--operands", default="normal",
                    help="input operand variant (workloads.OPERAND_VARIANTS): normal (the benchmark), "
                         "mant2 or paired_keys, for measuring data-dependent matrix-core throughput")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this S2-Attn build runs on one GPU only; no multi-GPU path exists "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from grouped_shifted_attention_amd import flops, ops

    name = args.workload or workloads.BENCH_WORKLOAD
    if name in workloads.LORA_WORKLOADS:
        return bench_lora(args, name)
    cfg = dict(workloads.WORKLOADS[name], name=name)
    rope = cfg["rope"]
    pattern = cfg.get("head_pattern", "second_half")
    fused = rope is not None or pattern != "second_half"
    B, N, H, Hkv, D, G, sh = (cfg[k] for k in ("B", "N", "H", "Hkv", "D", "G", "shift"))
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    x = workloads.make_inputs(B, N, H, Hkv, D, seed=0, operands=args.operands)
    to_gpu = lambda bits: torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v, do = (to_gpu(x[n]) for n in ("q", "k", "v", "dout"))
    out = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = ops.bwd_workspace(q, k, rope=rope is not None)
    ws_f = ops.fwd_rope_workspace(q, k) if rope is not None else None
    stream = torch.cuda.current_stream(dev)

    calib_copy(args, dev)

    kernels = ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"]
    if fused:
        # The general entry points have no stage calls: time the forward
        # (with its k rotation) and the backward (rotations or q scaling,
        # the statistics pass, dK/dV, dQ) as whole calls.
        kernels = ["fwd_call", "bwd_call"]

    def step_fused(events=None):
        if events is not None:
            events[0].record(stream)
        ops.s2attn_fwd_ex(q, k, v, G, sh, head_pattern=pattern, rope=rope, out=out, lse=lse, workspace=ws_f)
        if events is not None:
            events[1].record(stream)
        ops.s2attn_bwd_ex(q, k, v, out, lse, do, G, sh, head_pattern=pattern, rope=rope, dq=dq, dk=dk, dv=dv,
                          workspace=ws)
        if events is not None:
            events[2].record(stream)

    def step(events=None):
        if fused:
            return step_fused(events)
        if events is not None:
            events[0].record(stream)
        ops.s2attn_fwd(q, k, v, G, sh, out=out, lse=lse)
        if events is not None:
            events[1].record(stream)
        ops.s2attn_bwd_preprocess(out, do, lse, ws)
        if events is not None:
            events[2].record(stream)
        ops.s2attn_bwd_dkdv(q, k, v, do, G, sh, ws, dk=dk, dv=dv)
        if events is not None:
            events[3].record(stream)
        ops.s2attn_bwd_dq(q, k, v, do, G, sh, ws, dq=dq)
        if events is not None:
            events[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    kernel_ms = {kname: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) if evs else 0.0
                 for j, kname in enumerate(kernels)}
    f_fwd = flops.s2attn_fwd_flops(B, H, N, G, D)
    f_bwd = flops.s2attn_bwd_flops(B, H, N, G, D)
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12

    # MFMA work each kernel performs, in effective causal FLOPs per launch:
    # forward 2 products, dK/dV 4 (S, dP, dV, dK), dQ 3 (S, dP, dQ).
    unit = B * H * N * G * D
    kernel_flops = {"fwd": 2 * unit, "bwd_dkdv": 4 * unit, "bwd_dq": 3 * unit}
    if fused:
        kernel_flops = {"fwd_call": 2 * unit, "bwd_call": 7 * unit}
    dominant = max(kernel_flops, key=lambda kname: kernel_ms[kname])
    achieved = kernel_flops[dominant] / (kernel_ms[dominant] * 1e-3) / 1e12
    roofline = {
        "bound": "mfma", "kernel": dominant, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
        "avg_launch_ms": kernel_ms[dominant],
    }
    try:
        rec = json.load(open(TRAFFIC_FILE))
        if (rec.get("kernel") == dominant and rec.get("workload") == name
                and rec.get("source_sha256") == kernel_source_digest()):
            roofline["traffic"] = rec["traffic_bytes"]
            roofline["traffic_source"] = ("not measured in this run: FETCH_SIZE + WRITE_SIZE counter passes of a "
                                          "separate profiled run on the same kernel sources, " + rec.get("source", ""))
    except (OSError, ValueError, KeyError):
        pass

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "N": N, "H": H, "Hkv": Hkv, "D": D, "G": G, "shift": sh,
                   "rope": list(rope) if rope is not None else None, "head_pattern": pattern,
                   "parallelism": "single-gpu", "operands": args.operands},
        "pct_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd_tflops": f_fwd / (kernel_ms[kernels[0]] * 1e-3) / 1e12,
        "bwd_tflops": f_bwd / (sum(kernel_ms[kk] for kk in kernels[1:]) * 1e-3) / 1e12,
        "kernel_ms": kernel_ms,
        "roofline": roofline,
        "hbm_gbs_algorithmic": {
            "fwd": flops.fwd_algorithmic_bytes(B, N, H, Hkv, D) / (kernel_ms[kernels[0]] * 1e-3) / 1e9,
            "bwd": flops.bwd_algorithmic_bytes(B, N, H, Hkv, D)
            / (sum(kernel_ms[kk] for kk in kernels[1:]) * 1e-3) / 1e9,
            "peak": PEAK_HBM_GBS,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
