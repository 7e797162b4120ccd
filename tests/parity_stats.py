"""Turn the statistics the GPU parity checks record into a Markdown table.

    DLM_PARITY_STATS=stats.jsonl python -m pytest tests -m gpu ...
    python tests/parity_stats.py stats.jsonl profiles/parity_stats.md "<command>"

Each line of the input is one check (tests/gpu_util.py `record`): a bf16
check's element count, largest ulp distance to the oracle's once-rounded value,
how many elements were more than 2 ulp away and how many of those only the
near-zero floor (gamma_n + extra) * S admitted; an fp32 check's largest
relative error and the count above 1e-5 relative; and the drift reports of the
256-switch chains.  Checks are grouped by test (parametrised cases of one test
function are summed).
"""
from __future__ import annotations

import json
import sys
from collections import OrderedDict


def _group(test: str) -> str:
    # tests/test_x.py::test_name[param] -> test_x.py::test_name
    name = test.split("/")[-1]
    return name.split("[")[0]


def summarise(lines):
    bf, f32, drift = OrderedDict(), OrderedDict(), []
    for ln in lines:
        ln = ln.strip()
        if not ln:
            continue
        r = json.loads(ln)
        if r["kind"] == "drift":
            drift.append(r)
            continue
        key = _group(r["test"])
        if r["kind"] == "bf16":
            a = bf.setdefault(key, {"checks": 0, "n": 0, "max_ulp": 0, "n_gt2ulp": 0, "n_floor_only": 0,
                                    "n_exact": 0, "n_fail": 0})
            a["checks"] += 1
            for k in ("n", "n_gt2ulp", "n_floor_only", "n_exact", "n_fail"):
                a[k] += int(r.get(k, 0))
            a["max_ulp"] = max(a["max_ulp"], int(r["max_ulp"]))
        elif r["kind"] == "f32":
            a = f32.setdefault(key, {"checks": 0, "n": 0, "max_rel": 0.0, "n_rel_gt_1e-5": 0,
                                     "n_floor_only": 0, "n_fail": 0})
            a["checks"] += 1
            for k in ("n", "n_rel_gt_1e-5", "n_floor_only", "n_fail"):
                a[k] += int(r.get(k, 0))
            a["max_rel"] = max(a["max_rel"], float(r["max_rel"]))
    return bf, f32, drift


def markdown(bf, f32, drift, command: str) -> str:
    out = ["# Parity statistics of the GPU tests against the oracle", "",
           "Made by:", "", "```", command, "```", "",
           "bf16 outputs pass when their ulp distance (ordered bf16 line) to the oracle's once-rounded "
           "binary64 value is at most 2, or when |gpu - exact| <= (gamma_n + extra) * S, the near-zero "
           "floor (S = sum of the magnitudes of the element's terms, from the oracle). "
           "`> 2 ulp` counts the elements the first test rejects; `floor only` how many of those the "
           "floor admitted; `fail` what neither admitted (a failed test).", "",
           "## bf16 checks (T3)", "",
           "| test | checks | elements | exact | max ulp | > 2 ulp | floor only | fail |",
           "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for k, a in bf.items():
        out.append(f"| {k} | {a['checks']} | {a['n']:,} | {a['n_exact']:,} | {a['max_ulp']} | "
                   f"{a['n_gt2ulp']:,} | {a['n_floor_only']:,} | {a['n_fail']} |")
    tot = {k: sum(a[k] for a in bf.values()) for k in ("checks", "n", "n_exact", "n_gt2ulp", "n_floor_only",
                                                     "n_fail")}
    if bf:
        out.append(f"| **all** | {tot['checks']} | {tot['n']:,} | {tot['n_exact']:,} | "
                   f"{max(a['max_ulp'] for a in bf.values())} | {tot['n_gt2ulp']:,} | "
                   f"{tot['n_floor_only']:,} | {tot['n_fail']} |")
    out += ["", "## fp32 checks (T2)", "",
            "| test | checks | elements | max rel. error | rel. > 1e-5 | floor only | fail |",
            "|---|---:|---:|---:|---:|---:|---:|"]
    for k, a in f32.items():
        out.append(f"| {k} | {a['checks']} | {a['n']:,} | {a['max_rel']:.3g} | {a['n_rel_gt_1e-5']:,} | "
                   f"{a['n_floor_only']:,} | {a['n_fail']} |")
    out += ["", "## Drift after 256 switches (T4)", "",
            "Free-running chains of 256 in-place switches, against the exact merge of the final set "
            "(W0 + its deltas, rounded once); ulp distances per element.", "",
            "| chain | elements | GPU vs exact: median / p99 / max ulp | oracle vs exact: median / p99 / max ulp "
            "| GPU max err / ulp(0.02) | oracle max err / ulp(0.02) | GPU vs oracle > 2 ulp |",
            "|---|---:|---|---|---:|---:|---:|"]
    for r in drift:
        g, o = r["gpu_vs_exact_ulp"], r["oracle_vs_exact_ulp"]
        out.append(f"| {r['what']} | {r['n']:,} | {g['median']:g} / {g['p99']:g} / {g['max']} | "
                   f"{o['median']:g} / {o['p99']:g} / {o['max']} | {r['gpu_max_err_over_ulp(0.02)']:.4g} | "
                   f"{r['oracle_max_err_over_ulp(0.02)']:.4g} | {r['gpu_vs_oracle_gt2ulp']:,} |")
    return "\n".join(out) + "\n"


def main(argv):
    src, dst = argv[1], argv[2]
    command = argv[3] if len(argv) > 3 else ""
    with open(src) as f:
        bf, f32, drift = summarise(f.readlines())
    with open(dst, "w") as f:
        f.write(markdown(bf, f32, drift, command))


if __name__ == "__main__":
    main(sys.argv)
