"""Helpers for the GPU parity tests: tolerance checks against the binary64 oracle.

Tolerances (derived from the arithmetic; the stated bar is rel 1e-5 for fp32
and 2 bf16 ulp for bf16 with fp32 accumulation):
  gamma_n = n u / (1 - n u), u = 2^-24: forward error bound of an n-term fp32
            sum, scaled by S = the sum of the magnitudes of every term of the
            element's expression (the oracle returns S per element).
  fp32  : |gpu - exact| <= max(1e-5 |exact|, gamma_n S)
  bf16  : ulp distance (ordered bf16 line) to the oracle's once-rounded value
          <= 2, or |gpu - exact| <= (gamma_n + extra) S  (the near-zero floor,
          where a cancellation leaves fewer bits than the fp32 accumulation kept)
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

U32 = 2.0 ** -24

# Where the checks append their statistics, one JSON object per line (the
# report script tests/parity_stats.py turns them into a table).  Unset: not
# recorded.
STATS_ENV = "DLM_PARITY_STATS"


def record(kind: str, what: str, stats: dict):
    """Append one check's statistics to the file named by $DLM_PARITY_STATS."""
    path = os.environ.get(STATS_ENV)
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    line = json.dumps({"kind": kind, "test": test, "what": what, **stats})
    with open(path, "a") as f:
        f.write(line + "\n")


def gamma(n: int, u: float = U32) -> float:
    return n * u / (1.0 - n * u)


def bf16_ordered(t: torch.Tensor) -> np.ndarray:
    b = t.detach().cpu().contiguous().view(torch.int16).numpy().astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFF), b)


def ulp_dist_bf16(a: torch.Tensor, b: torch.Tensor) -> np.ndarray:
    return np.abs(bf16_ordered(a) - bf16_ordered(b))


def check_bf16(gpu, ref, exact, absum, n_terms, extra=0.0, what=""):
    """Compare bf16 results with the oracle; returns the statistics dict (also
    recorded, pass or fail, when $DLM_PARITY_STATS is set)."""
    d = ulp_dist_bf16(gpu, ref)
    err = np.abs(gpu.detach().cpu().double().numpy() - exact.numpy())
    floor = (gamma(n_terms) + extra) * absum.numpy()
    ok = (d <= 2) | (err <= floor)
    stats = {
        "n": int(d.size),
        "max_ulp": int(d.max()) if d.size else 0,
        "n_gt2ulp": int((d > 2).sum()),
        "n_floor_only": int(((d > 2) & (err <= floor)).sum()),
        "n_exact": int((d == 0).sum()),
        "n_fail": int((~ok).sum()),
    }
    record("bf16", what, stats)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        rows = [(tuple(int(i) for i in b), float(gpu.detach().cpu().double().numpy()[tuple(b)]),
                 float(exact.numpy()[tuple(b)]), int(d[tuple(b)]), float(floor[tuple(b)])) for b in bad]
        raise AssertionError(f"{what}: {int((~ok).sum())} elements out of tolerance; "
                             f"first (index, gpu, exact, ulp, floor): {rows}; stats {stats}")
    return stats


def check_f32(gpu, exact, absum, n_terms, what=""):
    g = gpu.detach().cpu().double().numpy()
    e = exact.numpy()
    err = np.abs(g - e)
    tol = np.maximum(1e-5 * np.abs(e), gamma(n_terms) * absum.numpy())
    ok = err <= tol
    stats = {"n": int(err.size),
             "max_rel": float((err / np.maximum(np.abs(e), 1e-30)).max()) if err.size else 0.0,
             "n_rel_gt_1e-5": int((err > 1e-5 * np.abs(e)).sum()),
             "n_floor_only": int(((err > 1e-5 * np.abs(e)) & ok).sum()),
             "n_fail": int((~ok).sum())}
    record("f32", what, stats)
    if not ok.all():
        b = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} out of tolerance, e.g. "
                             f"{[(tuple(map(int, i)), g[tuple(i)], e[tuple(i)]) for i in b]}")
    return stats


def host_set(idx_row, g_row):
    """(idx[2], g[2]) host lists from a row of CPU tensors."""
    return (list(map(int, idx_row.tolist())), list(map(float, g_row.tolist())))


def dev_set(s, device="cuda"):
    if s is None:
        return None
    return (torch.tensor(s[0], dtype=torch.int32, device=device),
            torch.tensor(s[1], dtype=torch.float32, device=device))


def sample_rows(d_out: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """First, last and k-2 random rows (sorted, unique)."""
    rows = {0, d_out - 1}
    if d_out > 2:
        rows.update(rng.choice(d_out, size=min(k, d_out) - len(rows) if k > 2 else 0,
                               replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
