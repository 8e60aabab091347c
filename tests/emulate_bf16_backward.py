"""Emulate, in float64 on the CPU, the bf16 and fp16 operand roundings of the
dK/dV kernel and measure how far they alone put its k/v gradients from the
fp64 oracle, on units of the 70B-style grouped-query shape (H 64, Hkv 8,
D 128, G 8192, RoPE base 1e4 with position interpolation 8).

Analysis script, not a test: it explains why the dK/dV kernel carries P to
the dS wave in fp16 and splits the operands of its diagonal products into
bf16 hi + lo.  Each k/v gradient sums the H/Hkv = 8 q heads that share the
k/v head, so its rounding error grows with the sharing; the bar it must meet
is max-abs 2e-2 beyond the output's own bf16 half-ulp.

What the emulation rounds, as the kernels do: q * log2(e)/sqrt(D) (after the
rotation) and k to bf16 once; the forward's P to bf16 before P V and its
output to bf16 (Delta = rowsum(dO * O)); in the backward P to bf16 for dV,
P to the hand-over format for dS = P (dP - Delta), and dS to bf16 for dK.
Sums are exact (float64), which is where the emulation differs from the
kernel (fp32 accumulation).  Gradients stay in the rotated frame on both
sides.  Keys 0 .. kmax-1 of each unit (the first key tiles, whose diagonal
and dense rows see every q row of the group) are compared.

Usage:  python tests/emulate_bf16_backward.py [--units all|first] [--kmax 256]
"""
from __future__ import annotations

import argparse
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402
from oracle import s2attn_ref  # noqa: E402

LOG2E = 1.4426950408889634
G, N, H, HKV, D, SHIFT, ROPE = 8192, 32768, 64, 8, 128, 4096, (10000.0, 8.0)


def bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), via fp32."""
    x = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def split_bf16(x):
    """bf16 hi + bf16 lo: the operand of a product taken as two MFMAs."""
    hi = bf16(x)
    return hi + bf16(x - hi)


def emulated_dkdv(qg, kg, vg, dog, scale, kmax, handover, split_diag):
    """dk, dv of keys [0, kmax) of one unit with the kernels' roundings.

    handover: the format P reaches the dS product in ('bf16' or 'fp16').
    split_diag: whether the dV and dK products of the 32 x 32 diagonal blocks
    take their operand as bf16 hi + lo."""
    G_, D_ = qg.shape
    qop, kop = bf16(qg * scale * LOG2E), bf16(kg)
    blk = 1024
    cols = np.arange(G_)[None, :]
    o = np.empty((G_, D_))
    lse2 = np.empty(G_)
    for r0 in range(0, G_, blk):  # forward: lse in log2 units, out rounded to bf16
        r1 = min(G_, r0 + blk)
        rows = np.arange(r0, r1)[:, None]
        s = np.where(cols <= rows, qop[r0:r1] @ kop.T, -np.inf)
        m = s.max(1, keepdims=True)
        e = np.exp2(s - m)
        z = e.sum(1, keepdims=True)
        o[r0:r1] = (bf16(e) @ vg) / z
        lse2[r0:r1] = (m + np.log2(z))[:, 0]
    delta = (dog * bf16(o)).sum(1)
    dk = np.zeros((kmax, D_))
    dv = np.zeros((kmax, D_))
    kc = np.arange(kmax)[None, :]
    for r0 in range(0, G_, blk):
        r1 = min(G_, r0 + blk)
        rows = np.arange(r0, r1)[:, None]
        p = np.where(kc <= rows, np.exp2(qop[r0:r1] @ kop[:kmax].T - lse2[r0:r1, None]), 0.0)
        diag = (rows // 32) == (kc // 32)
        p_dv = np.where(diag, split_bf16(p), bf16(p)) if split_diag else bf16(p)
        p_ds = fp16(p) if handover == "fp16" else bf16(p)
        ds = p_ds * (dog[r0:r1] @ vg[:kmax].T - delta[r0:r1, None])
        ds_dk = np.where(diag, split_bf16(ds), bf16(ds)) if split_diag else bf16(ds)
        dv += p_dv.T @ dog[r0:r1]
        dk += (ds_dk.T @ qop[r0:r1]) * math.log(2)
    return dk, dv


def beyond_rounding(got, ref):
    """max |bf16(got) - ref| minus each element's bf16 half-ulp |ref| 2^-8."""
    return float(np.max(np.abs(bf16(got) - ref) - 2.0 ** -8 * np.abs(ref)))


VARIANTS = {
    "bf16 P hand-over, no diagonal split": ("bf16", False),
    "fp16 P hand-over, no diagonal split": ("fp16", False),
    "fp16 P hand-over + hi/lo diagonal (the kernel)": ("fp16", True),
}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--units", default="first", choices=["first", "all"],
                    help="first: k/v head 0, group 0; all: k/v heads {0, 3, 4, 7} x groups {0, 3}")
    ap.add_argument("--kmax", type=int, default=256)
    args = ap.parse_args()
    units = [(0, 0)] if args.units == "first" else [(kv, g) for kv in (0, 3, 4, 7) for g in (0, 3)]
    print("generating the seeded inputs", flush=True)
    x = workloads.make_inputs(1, N, H, HKV, D, seed=0)
    rq = H // HKV
    worst = {name: [0.0, 0.0] for name in VARIANTS}
    for kvh, g in units:
        t0 = time.time()
        ref = [np.zeros((args.kmax, D)), np.zeros((args.kmax, D))]
        acc = {name: [np.zeros((args.kmax, D)), np.zeros((args.kmax, D))] for name in VARIANTS}
        for h in range(kvh * rq, (kvh + 1) * rq):
            f64 = lambda name, hh: workloads.f64_from_bf16_bits(x[name][0, :, hh, :])
            sh = oracle.head_shift(h, H, SHIFT, "second_half", HKV)
            (qg, kg, vg, dog), _, scale = s2attn_ref._head_unit_operands(
                f64("q", h), f64("k", kvh), f64("v", kvh), f64("dout", h), G, sh, g, ROPE)
            _, dkr, dvr = oracle.group_causal_attention_backward(qg, kg, vg, dog, scale)
            ref[0] += dkr[:args.kmax]
            ref[1] += dvr[:args.kmax]
            for name, (handover, split) in VARIANTS.items():
                dk, dv = emulated_dkdv(qg, kg, vg, dog, scale, args.kmax, handover, split)
                acc[name][0] += dk
                acc[name][1] += dv
        print(f"unit k/v head {kvh}, group {g} ({time.time() - t0:.0f} s):")
        for name in VARIANTS:
            ek, ev = beyond_rounding(acc[name][0], ref[0]), beyond_rounding(acc[name][1], ref[1])
            worst[name] = [max(worst[name][0], ek), max(worst[name][1], ev)]
            print(f"  {name:48s} dk {ek:.3e}  dv {ev:.3e}  (beyond bf16 rounding; bar 2e-2)")
    if len(units) > 1:
        print("worst over the units:")
        for name, (ek, ev) in worst.items():
            print(f"  {name:48s} dk {ek:.3e}  dv {ev:.3e}")


if __name__ == "__main__":
    main()
