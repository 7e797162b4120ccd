"""Brute-force re-derivations for tiny sizes (NumPy, binary64).

TEST INFRASTRUCTURE ONLY, like oracle.c, and written independently of it: the
router enumerates every ordered expert pair instead of scanning for maxima, and
the adapter products use NumPy's matmul on whole matrices instead of
element-by-element loops.  All results are unrounded binary64.
"""
from __future__ import annotations

import itertools

import numpy as np


def f64(t):
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to(torch.float64).cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def pregate(x, Wr):
    """Top-2 by exhaustive search over ordered pairs (i, j), i != j.

    The chosen pair maximises l_i first and l_j second; among equal logits the
    lower index wins, i.e. the key (-l_i, i, -l_j, j) is minimal.  Weights are
    exp(l_i)/(exp(l_i)+exp(l_j)) and exp(l_j)/(...), the two-way renormalised
    softmax.  Returns idx [T][2], g [T][2] (binary64), logits [T][E]."""
    x = f64(x)
    Wr = f64(Wr)
    T, d = x.shape
    E = Wr.shape[1]
    logits = np.zeros((T, E))
    for t in range(T):
        for e in range(E):
            logits[t, e] = sum(x[t, j] * Wr[j, e] for j in range(d))
    idx = np.zeros((T, 2), np.int64)
    g = np.zeros((T, 2))
    for t in range(T):
        l = logits[t]
        best = min(itertools.permutations(range(E), 2),
                   key=lambda p: (-l[p[0]], p[0], -l[p[1]], p[1]))
        idx[t] = best
        m = max(l[best[0]], l[best[1]])
        a, b = np.exp(l[best[0]] - m), np.exp(l[best[1]] - m)
        g[t] = (a / (a + b), b / (a + b))
    return idx, g, logits


def set_delta_matrix(A, B, s, st):
    """s * sum_k g_k * (B[e_k] @ A[e_k]) for a set st = (idx, g) or None."""
    A = f64(A)
    B = f64(B)
    d_out, d_in = B.shape[1], A.shape[2]
    D = np.zeros((d_out, d_in))
    if st is None:
        return D
    ids, gs = st
    for e, gk in zip(np.asarray(ids).reshape(-1), np.asarray(gs, dtype=np.float64).reshape(-1)):
        if e < 0:
            continue
        D += s * gk * (B[e] @ A[e])
    return D


def switch(W, A, B, s, old, new):
    """Unrounded W - delta(old) + delta(new) with whole-matrix products."""
    return f64(W) - set_delta_matrix(A, B, s, old) + set_delta_matrix(A, B, s, new)


def sgmm(x, idx, g, A, B, y, s):
    """Unrounded y + sum_k s g_k B[e_k] (A[e_k] x_t) per row with matrix-vector products."""
    x, A, B, y = f64(x), f64(A), f64(B), f64(y)
    idx = np.asarray(idx).reshape(-1, 2)
    g = np.asarray(g, dtype=np.float64).reshape(-1, 2)
    out = y.copy()
    for t in range(x.shape[0]):
        for k in range(2):
            e = int(idx[t, k])
            if e < 0:
                continue
            out[t] += s * g[t, k] * (B[e] @ (A[e] @ x[t]))
    return out
