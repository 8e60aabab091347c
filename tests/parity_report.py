"""Render the parity margins a GPU test run logged into a Markdown table.

The GPU parity tests append one JSON line per compared tensor to the file
named by S2A_PARITY_LOG (see gpu_helpers.log_margin).  Usage:

    S2A_PARITY_LOG=gpurun_out/parity_log.jsonl python -m pytest tests -m gpu
    python tests/parity_report.py gpurun_out/parity_log.jsonl > profiles/parity_margins.md
"""
import json
import sys


def main(path, command=None):
    rows = [json.loads(l) for l in open(path) if l.strip()]
    lines = ["# Parity margins of the GPU tests against the fp64 oracle", ""]
    if command:
        lines += ["Command (from the repository root on the GPU box):", "", "```", command, "```", ""]
    n_over = sum(r["beyond_rounding"] > r["bar_max_abs"] or r["rel_l2"] > r["bar_rel_l2"] for r in rows)
    lines += [
        f"{len(rows)} compared tensors; {n_over} outside their bar.  `beyond rounding` is "
        "max |gpu - oracle| minus each element's own output half-ulp (|oracle| 2^-8 for bf16 tensors, 0 for "
        "the fp32 log-sum-exp), the quantity held to max-abs 2e-2; `plain` is max |gpu - oracle|; `rel-L2` is "
        "||gpu - oracle|| / ||oracle|| (bar 1e-2).  `margin` = beyond rounding / bar.",
        "",
        "One row per test function and tensor kind, the worst over its parametrised cases and sampled units.",
        "",
        "| test | tensor | comparisons | worst beyond rounding | worst plain max-abs | worst rel-L2 | margin |",
        "|---|---|---:|---:|---:|---:|---:|",
    ]
    groups = {}
    for r in rows:
        fn = r["test"].split("::")[-1].split("[")[0]
        kind = r["tensor"].split("[")[0].split("(")[0]
        groups.setdefault((fn, kind), []).append(r)
    for (fn, kind), rs in groups.items():
        b = max(x["beyond_rounding"] for x in rs)
        margin = max(x["beyond_rounding"] / x["bar_max_abs"] for x in rs)
        lines.append(f"| `{fn}` | {kind} | {len(rs)} | {b:.2e} | {max(x['plain_max_abs'] for x in rs):.2e} | "
                     f"{max(x['rel_l2'] for x in rs):.2e} | {margin:.2f} |")
    worst = sorted(rows, key=lambda r: -r["beyond_rounding"] / r["bar_max_abs"])[:10]
    lines += ["", "Closest to the bar:", ""]
    for r in worst:
        lines.append(f"- `{r['test'].split('::', 1)[-1]}` {r['tensor']}: {r['beyond_rounding']:.2e} beyond "
                     f"rounding (bar {r['bar_max_abs']:g}), rel-L2 {r['rel_l2']:.2e}")
    print("\n".join(lines))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else None)
