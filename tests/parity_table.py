"""Turns the JSON-lines parity record of a GPU test run into a markdown table.

    LM_PARITY_RECORD=<file> python -m pytest tests -m gpu ...
    python tests/parity_table.py <file> [--all] > profiles/parity_margins.md

Each row is one comparison of the HIP path with the fp64 oracle: the metric the
test applies (float32 inputs: max-rel = max|x - r| / max|r|; bf16 inputs:
rel-L2 = ||x - r|| / ||r||), its value, the tolerance and the margin
(tolerance / value). By default only the whole-tensor checks of the full-size
workloads and the CCQ sensitivity lines are listed, plus a summary of the rest.
"""
from __future__ import annotations

import argparse
import json
import math
import sys


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("record")
    ap.add_argument("--all", action="store_true", help="list every comparison")
    args = ap.parse_args()
    rows = [json.loads(l) for l in open(args.record) if l.strip()]
    checks = [r for r in rows if not math.isnan(r["tol"])]
    sens = [r for r in rows if math.isnan(r["tol"])]

    def full(r):
        return args.all or "whole tensor" in r["what"] or "(ccq_bf16" in r["what"]

    out = sys.stdout
    out.write("| check | metric | value | tolerance | margin |\n|---|---|---|---|---|\n")
    for r in checks:
        if full(r):
            out.write("| %s | %s | %.3e | %.0e | %.0fx |\n" % (r["what"], r["metric"], r["value"], r["tol"],
                                                          r["tol"] / max(r["value"], 1e-300)))
    rest = [r for r in checks if not full(r)]
    if rest and not args.all:
        for metric in sorted({r["metric"] for r in rest}):
            sub = [r for r in rest if r["metric"] == metric]
            worst = max(sub, key=lambda r: r["value"] / r["tol"])
            out.write("\nOther %s checks: %d, largest %.3e (tolerance %.0e) at \"%s\" (%s).\n"
                      % (metric, len(sub), worst["value"], worst["tol"], worst["what"], worst["test"]))
    if sens:
        out.write("\nSensitivity (oracle only): rel-L2 between the CCQ and the plain decayed read on the "
                  "same inputs, i.e. how much of the output the covariance correction moves.\n\n"
                  "| inputs | rel-L2 CCQ vs GLA |\n|---|---|\n")
        seen = set()
        for r in sens:
            key = (r["what"], round(r["value"], 6))
            if key in seen:
                continue
            seen.add(key)
            out.write("| %s | %.3e |\n" % (r["what"].replace("oracle CCQ vs GLA at ", ""), r["value"]))


if __name__ == "__main__":
    main()
