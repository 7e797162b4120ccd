"""Pins of the CPU oracle against things other than itself.

Each pin takes an oracle library handle, so the same checks run on the real
oracle (they must all pass) and on copies with a planted mistake (at least one
must fail).  What each pin holds the oracle to:

  golden    hand-worked examples (tests/golden/*.json, each with its derivation)
  brute     oracle/brute.py: exhaustive pair search, NumPy whole-matrix products
  closed    closed forms: two-logit softmax = logistic of the logit gap
  premerge  switch from the empty set = W + s*sum g B@A (static pre-merge)
  noop      a switch to the same set leaves W bitwise unchanged
  roundtrip A -> B -> A returns the starting weights within the rounding bound
  merged    merged weights applied to x = base output + unmerged adapters
  gemm      SGMM with one set for every row = a dense textbook GEMM
  centroid  nearest-centroid router: hand-worked fixture, NumPy brute force,
            permutation / translation / duplicate invariants
  gemv      merged-weight product against NumPy's binary64 matmul; merged
            product = base product + unmerged adapters + the rounding of W
  absum     the tolerance scale S each output carries (the sum of the
            magnitudes of every term of its expression), recomputed from both
            sides with NumPy whole-matrix products of absolute values; the
            router's bound gamma_d * max_e sum_j |x_j Wr_je| the same way
  rounding  one nearest-even rounding to bf16 / fp32
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _t(v, dtype):
    return torch.tensor(v, dtype=torch.float64).to(dtype)


def _set(s):
    if s is None:
        return None
    return (list(s[0]), [float(x) for x in s[1]])


def _rng(seed):
    return np.random.default_rng(seed)


def _dyadic(rng, shape, scale=4, den=4):
    """Small dyadic rationals: exact in bf16/fp32 and in sums of a few products."""
    return rng.integers(-scale * den, scale * den + 1, size=shape).astype(np.float64) / den


def _fp32_ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


# ---------------------------------------------------------------- router ----

def pin_router_golden(lib):
    for c in _golden("router_tiny.json")["cases"]:
        for dt in (torch.float32, torch.bfloat16):
            idx, g = oracle.pregate(_t(c["x"], dt), _t(c["Wr"], dt), lib=lib)
            assert idx.tolist() == c["idx"], (c["note"], idx.tolist())
            want = np.asarray(c["g"], np.float64).astype(np.float32)
            assert (_fp32_ulps(g.numpy(), want) <= 1).all(), (c["note"], g, want)


def pin_router_brute(lib):
    rng = _rng(11)
    for trial in range(60):
        E = int(rng.integers(2, 7))
        d = int(rng.integers(1, 6))
        T = int(rng.integers(1, 5))
        # coarse values make exact ties frequent
        x = _dyadic(rng, (T, d), scale=2, den=2)
        Wr = _dyadic(rng, (d, E), scale=2, den=2)
        for dt in (torch.float32, torch.bfloat16):
            idx, g = oracle.pregate(_t(x, dt), _t(Wr, dt), lib=lib)
            bi, bg, _ = brute.pregate(x, Wr)
            assert (idx.numpy() == bi).all(), (trial, x, Wr, idx, bi)
            assert (_fp32_ulps(g.numpy(), bg.astype(np.float32)) <= 1).all(), (trial, g, bg)


def pin_router_closed_form(lib):
    rng = _rng(12)
    T, d, E = 64, 32, 8
    x = torch.from_numpy(rng.standard_normal((T, d))).float()
    Wr = torch.from_numpy(rng.standard_normal((d, E)) * 0.3).float()
    idx, g, lg, mg, bd = oracle.pregate(x, Wr, with_stats=True, lib=lib)
    # logits are the matrix product (the products of fp32 values are exact in binary64)
    ref_l = x.double() @ Wr.double()
    assert torch.allclose(lg, ref_l, rtol=0, atol=1e-12)
    l = lg.numpy()
    i = idx.numpy().astype(np.int64)
    l0 = l[np.arange(T), i[:, 0]]
    l1 = l[np.arange(T), i[:, 1]]
    assert (l0 >= l1).all() and (i[:, 0] != i[:, 1]).all()
    # slot 0 is the maximum, slot 1 the maximum of the rest
    assert np.allclose(l0, l.max(1), rtol=0, atol=0)
    masked = l.copy()
    masked[np.arange(T), i[:, 0]] = -np.inf
    assert np.allclose(l1, masked.max(1), rtol=0, atol=0)
    g0 = (1.0 / (1.0 + np.exp(l1 - l0))).astype(np.float32)
    g1 = (np.exp(l1 - l0) / (1.0 + np.exp(l1 - l0))).astype(np.float32)
    assert (_fp32_ulps(g.numpy()[:, 0], g0) <= 1).all()
    assert (_fp32_ulps(g.numpy()[:, 1], g1) <= 1).all()
    assert (g.numpy()[:, 0] >= g.numpy()[:, 1]).all()
    assert np.abs(g.double().sum(1).numpy() - 1.0).max() <= 2 ** -23
    # margin = distance of the decision from a tie
    srt = np.sort(l, 1)[:, ::-1]
    assert np.allclose(mg.numpy(), np.minimum(srt[:, 0] - srt[:, 1], srt[:, 1] - srt[:, 2]))
    assert (bd.numpy() > 0).all() and (bd.numpy() < 1e-12).all()


def pin_router_permutation(lib):
    rng = _rng(13)
    T, d, E = 32, 16, 6
    x = torch.from_numpy(rng.standard_normal((T, d))).float()
    Wr = torch.from_numpy(rng.standard_normal((d, E))).float()
    idx, g = oracle.pregate(x, Wr, lib=lib)
    perm = rng.permutation(E)
    idx2, g2 = oracle.pregate(x, Wr[:, perm].contiguous(), lib=lib)
    # column c of the permuted router is expert perm[c]
    assert (perm[idx2.numpy()] == idx.numpy()).all()
    assert torch.equal(g, g2)
    # duplicated columns give identical logits: the lower index always wins, so
    # expert 4 (a copy of 1) is only ever chosen as (1, 4)
    Wd = Wr.clone()
    Wd[:, 4] = Wd[:, 1]
    idx3, g3 = oracle.pregate(x, Wd, lib=lib)
    seen = 0
    for t in range(T):
        p = idx3[t].tolist()
        if 4 in p:
            assert p == [1, 4] and g3[t, 0].item() == 0.5, p
            seen += 1
    assert (idx3 == 1).any()
    # force the tie into the top two for one token and check it is resolved
    x2 = torch.zeros(1, d)
    x2[0, 0] = 1.0
    Wt = torch.zeros(d, E)
    Wt[0, 1] = Wt[0, 4] = 3.0
    Wt[0, 0] = 1.0
    assert oracle.pregate(x2, Wt, lib=lib)[0].tolist() == [[1, 4]]


# ------------------------------------------------------ centroid router ----

def pin_centroid_golden(lib):
    c = _golden("centroid_tiny.json")
    for dt in (torch.float32, torch.bfloat16):
        idx, g, dist, _ = oracle.pregate_centroid(_t(c["x"], dt), _t(c["C"], dt), with_stats=True, lib=lib)
        assert idx.tolist() == c["idx"] and g.tolist() == c["g"], (idx, g)
        assert dist.tolist() == c["dist"], dist


def _centroid_brute(x, C):
    X, Cd = x.double().numpy(), C.double().numpy()
    d2 = ((X[:, None, None, :] - Cd[None]) ** 2).sum(-1)    # [T][E][J]
    de = d2.min(-1)
    return de, de.argmin(-1)                                  # first minimum: lower index on ties


def pin_centroid_brute(lib):
    rng = _rng(51)
    for dt in (torch.float32, torch.bfloat16):
        for T, d, E, J in ((1, 1, 1, 1), (9, 5, 3, 2), (17, 33, 8, 4), (5, 64, 16, 1)):
            x = torch.from_numpy(rng.standard_normal((T, d))).to(dt)
            C = torch.from_numpy(rng.standard_normal((E, J, d))).to(dt)
            idx, g, dist, mg = oracle.pregate_centroid(x, C, with_stats=True, lib=lib)
            de, eb = _centroid_brute(x, C)
            assert np.allclose(dist.numpy(), de, rtol=1e-13, atol=0)
            assert (idx[:, 0].numpy() == eb).all() and (idx[:, 1] == -1).all()
            assert (g[:, 0] == 1).all() and (g[:, 1] == 0).all()
            srt = np.sort(de, axis=1)
            ref_m = srt[:, 1] - srt[:, 0] if E > 1 else np.full(T, np.inf)
            assert np.allclose(mg.numpy(), ref_m, rtol=1e-12, atol=1e-12)


def pin_centroid_invariants(lib):
    rng = _rng(52)
    T, d, E, J = 12, 16, 6, 3
    x = torch.from_numpy(_dyadic(rng, (T, d))).float()
    C = torch.from_numpy(_dyadic(rng, (E, J, d))).float()
    idx, _, dist, _ = oracle.pregate_centroid(x, C, with_stats=True, lib=lib)
    # permuting adapters permutes the choice (ties aside: none at these seeds)
    perm = rng.permutation(E)
    idx_p, _, dist_p, _ = oracle.pregate_centroid(x, C[perm], with_stats=True, lib=lib)
    assert torch.equal(dist_p, dist[:, perm])
    assert (perm[idx_p[:, 0].numpy()] == idx[:, 0].numpy()).all()
    # permuting an adapter's own centroids changes nothing
    idx_j, _, dist_j, _ = oracle.pregate_centroid(x, C[:, rng.permutation(J)], with_stats=True, lib=lib)
    assert torch.equal(idx_j, idx) and torch.equal(dist_j, dist)
    # translating x and every centroid by the same (dyadic) vector changes nothing
    sh = torch.from_numpy(_dyadic(rng, (d,))).float()
    idx_t, _, dist_t, _ = oracle.pregate_centroid(x + sh, C + sh, with_stats=True, lib=lib)
    assert torch.equal(idx_t, idx) and torch.equal(dist_t, dist)
    # a token sitting on a centroid of adapter e picks e (distance 0) unless a lower adapter also has 0
    x0 = C[4, 1].reshape(1, d).clone()
    i0, _, d0, _ = oracle.pregate_centroid(x0, C, with_stats=True, lib=lib)
    assert d0[0, 4] == 0 and i0[0, 0] == 4
    # an adapter duplicated at a higher index never wins over its original
    C2 = torch.cat([C, C[2:3]], 0)
    i2, _, _, _ = oracle.pregate_centroid(x, C2, with_stats=True, lib=lib)
    assert (i2[:, 0] != E).all()


# ---------------------------------------------------------------- switch ----

def pin_switch_golden(lib):
    for c in _golden("switch_tiny.json")["cases"]:
        dt = torch.float32 if c["dtype"] == "fp32" else torch.bfloat16
        W = _t(c["W0"], dt)
        A = _t(c["A"], dt)
        B = _t(c["B"], dt)
        for st in c["steps"]:
            W = oracle.switch(W, A, B, c["scale"], _set(st["old"]), _set(st["new"]), lib=lib)
            assert torch.equal(W, _t(st["W"], dt)), (c["dtype"], st, W)


def _rand_bank(rng, E, r, d_in, d_out, dt):
    A = torch.from_numpy(rng.standard_normal((E, r, d_in)) * 0.5).to(dt)
    B = torch.from_numpy(rng.standard_normal((E, d_out, r)) * 0.5).to(dt)
    return A, B


def _rand_set(rng, E, allow_empty=True):
    e = rng.choice(E, size=2, replace=E < 2)
    if allow_empty and rng.random() < 0.2:
        e[1] = -1
    g = rng.random(2).astype(np.float32)
    return (e.tolist(), g.tolist())


def pin_switch_premerge(lib):
    rng = _rng(21)
    for trial in range(12):
        E, r = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        d_out, d_in = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        s = float(rng.choice([1.0, 2.0, 0.5]))
        for dt in (torch.float32, torch.bfloat16):
            A, B = _rand_bank(rng, E, r, d_in, d_out, dt)
            W0 = torch.from_numpy(rng.standard_normal((d_out, d_in))).to(dt)
            S = _rand_set(rng, E)
            W1, ex, _ = oracle.switch(W0, A, B, s, None, S, with_stats=True, lib=lib)
            ref = brute.switch(W0, A, B, s, None, S)
            assert np.allclose(ex.numpy(), ref, rtol=1e-12, atol=1e-12), (trial, ex, ref)
            # the stored result is the once-rounded exact value
            rr = oracle.round_to(ref, 0 if dt == torch.float32 else 1, lib=oracle.load())
            got = W1.numpy() if dt == torch.float32 else W1.view(torch.int16).numpy().view(np.uint16)
            assert (got == rr).all(), (trial, got, rr)


def pin_switch_general(lib):
    rng = _rng(22)
    for trial in range(12):
        E, r = int(rng.integers(2, 5)), int(rng.integers(1, 5))
        d_out, d_in = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        s = float(rng.choice([1.0, 2.0]))
        A, B = _rand_bank(rng, E, r, d_in, d_out, torch.float32)
        W0 = torch.from_numpy(rng.standard_normal((d_out, d_in))).float()
        old, new = _rand_set(rng, E), _rand_set(rng, E)
        _, ex, ab = oracle.switch(W0, A, B, s, old, new, with_stats=True, lib=lib)
        ref = brute.switch(W0, A, B, s, old, new)
        assert np.allclose(ex.numpy(), ref, rtol=1e-12, atol=1e-12)
        # the magnitude sum bounds the value and includes |W|
        assert (ab.numpy() + 1e-12 >= np.abs(ref)).all()
        assert (ab.numpy() + 1e-12 >= np.abs(W0.double().numpy())).all()


def pin_switch_noop(lib):
    rng = _rng(23)
    for dt in (torch.float32, torch.bfloat16):
        E, r, d_out, d_in = 4, 3, 7, 9
        A, B = _rand_bank(rng, E, r, d_in, d_out, dt)
        W0 = torch.from_numpy(rng.standard_normal((d_out, d_in))).to(dt)
        S = ([2, 0], [0.7, 0.3])
        assert torch.equal(oracle.switch(W0, A, B, 2.0, S, S, lib=lib), W0)
        swapped = ([0, 2], [0.3, 0.7])
        assert torch.equal(oracle.switch(W0, A, B, 2.0, S, swapped, lib=lib), W0)
        assert torch.equal(oracle.switch(W0, A, B, 2.0, None, None, lib=lib), W0)


def pin_switch_roundtrip(lib):
    rng = _rng(24)
    E, r, d_out, d_in = 4, 4, 16, 16
    for dt, tol_rel in ((torch.float32, 1e-6), (torch.bfloat16, None)):
        A, B = _rand_bank(rng, E, r, d_in, d_out, dt)
        W0 = torch.from_numpy(rng.standard_normal((d_out, d_in))).to(dt)
        SA, SB = ([0, 1], [0.6, 0.4]), ([3, 2], [0.8, 0.2])
        WA = oracle.switch(W0, A, B, 1.0, None, SA, lib=lib)
        WB = oracle.switch(WA, A, B, 1.0, SA, SB, lib=lib)
        WA2 = oracle.switch(WB, A, B, 1.0, SB, SA, lib=lib)
        W02 = oracle.switch(WA2, A, B, 1.0, SA, None, lib=lib)
        a, b, mid = WA.double(), WA2.double(), WB.double()
        if tol_rel is not None:
            scale = a.abs() + mid.abs()
            assert ((a - b).abs() <= tol_rel * scale + 1e-30).all()
            assert ((W0.double() - W02.double()).abs() <= tol_rel * (W0.double().abs() + mid.abs())).all()
        else:
            # each of the two switches rounds once: the difference is bounded by half a
            # bf16 spacing of the intermediate plus half a spacing of the result
            def sp(v):
                m, e = np.frexp(np.abs(v.numpy()))
                return np.ldexp(1.0, e - 8)
            bound = 0.5 * sp(mid) + 0.5 * sp(b)
            assert (np.abs((a - b).numpy()) <= bound + 1e-30).all()


def pin_merged_equals_unmerged(lib):
    rng = _rng(25)
    E, r, d_out, d_in, T = 3, 4, 6, 10, 5
    A, B = _rand_bank(rng, E, r, d_in, d_out, torch.float32)
    W0 = torch.from_numpy(rng.standard_normal((d_out, d_in))).float()
    x = torch.from_numpy(rng.standard_normal((T, d_in))).float()
    S = ([2, 0], [0.625, 0.375])
    _, Wm, _ = oracle.switch(W0, A, B, 2.0, None, S, with_stats=True, lib=lib)
    idx = torch.tensor([S[0]] * T, dtype=torch.int32)
    g = torch.tensor([S[1]] * T, dtype=torch.float32)
    y0 = torch.zeros(T, d_out)
    _, ys, _ = oracle.sgmm(x, idx, g, A, B, y0, 2.0, with_stats=True, lib=lib)
    lhs = x.double().numpy() @ Wm.numpy().T
    rhs = x.double().numpy() @ W0.double().numpy().T + ys.numpy()
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def pin_switch_absum(lib):
    """S of a switched element = |W| + sum over both sets' used slots of
    |s g_k| * (|B_e| @ |A_e|): equal both ways (not only a lower bound), so a
    wrong S cannot widen or narrow the parity floor unnoticed."""
    rng = _rng(26)
    for trial in range(10):
        E, r = int(rng.integers(1, 5)), int(rng.integers(1, 6))
        d_out, d_in = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        s = float(rng.choice([1.0, 2.0, 0.5, -1.5]))
        for dt in (torch.float32, torch.bfloat16):
            A, B = _rand_bank(rng, E, r, d_in, d_out, dt)
            W0 = torch.from_numpy(rng.standard_normal((d_out, d_in))).to(dt)
            old = None if trial % 4 == 0 else _rand_set(rng, E)
            new = None if trial % 4 == 1 else _rand_set(rng, E)
            _, _, ab = oracle.switch(W0, A, B, s, old, new, with_stats=True, lib=lib)
            Ad, Bd = np.abs(A.double().numpy()), np.abs(B.double().numpy())
            ref = np.abs(W0.double().numpy()).copy()
            for st in (old, new):
                if st is None:
                    continue
                for e, gk in zip(st[0], st[1]):
                    if e >= 0:
                        ref += abs(s * float(np.float32(gk))) * (Bd[e] @ Ad[e])
            assert np.allclose(ab.numpy(), ref, rtol=1e-12, atol=0), (trial, ab, ref)


def pin_router_bound(lib):
    """The router's decision bound = gamma_d(2^-53) * max_e sum_j |x_j Wr_je|."""
    rng = _rng(14)
    for T, d, E in ((5, 1, 2), (17, 33, 8), (9, 300, 5)):
        x = torch.from_numpy(rng.standard_normal((T, d))).float()
        Wr = torch.from_numpy(rng.standard_normal((d, E)) * 0.3).float()
        _, _, _, _, bd = oracle.pregate(x, Wr, with_stats=True, lib=lib)
        u = 2.0 ** -53
        gam = d * u / (1.0 - d * u)
        ref = gam * (np.abs(x.double().numpy()) @ np.abs(Wr.double().numpy())).max(1)
        assert np.allclose(bd.numpy(), ref, rtol=1e-12, atol=0), (bd, ref)


# ------------------------------------------------------------------ gemv ----

def pin_gemv_golden(lib):
    for c in _golden("gemv_tiny.json")["cases"]:
        dt = torch.float32 if c["dtype"] == "fp32" else torch.bfloat16
        y = oracle.gemv(_t(c["W"], dt), _t(c["x"], dt), lib=lib)
        assert torch.equal(y, torch.tensor(c["y"], dtype=torch.float32)), (c, y)


def pin_gemv_numpy(lib):
    rng = _rng(41)
    for dt in (torch.float32, torch.bfloat16):
        for d_out, d_in in ((1, 1), (7, 13), (33, 257)):
            W = torch.from_numpy(rng.standard_normal((d_out, d_in))).to(dt)
            x = torch.from_numpy(rng.standard_normal(d_in)).to(dt)
            y, ex, ab = oracle.gemv(W, x, with_stats=True, lib=lib)
            ref = W.double().numpy() @ x.double().numpy()
            assert np.allclose(ex.numpy(), ref, rtol=1e-12, atol=1e-12 * ab.numpy().max())
            assert np.allclose(ab.numpy(), np.abs(W.double().numpy()) @ np.abs(x.double().numpy()), rtol=1e-12)
            assert (_fp32_ulps(y.numpy(), ref.astype(np.float32)) <= 1).all()


def pin_gemv_merged(lib):
    """Product with the merged (rounded) weight = base product + unmerged
    adapters + x applied to the rounding of the merged weight."""
    rng = _rng(42)
    E, r, d_out, d_in = 4, 3, 9, 21
    for dt in (torch.float32, torch.bfloat16):
        A, B = _rand_bank(rng, E, r, d_in, d_out, dt)
        W0 = torch.from_numpy(rng.standard_normal((d_out, d_in))).to(dt)
        x = torch.from_numpy(rng.standard_normal(d_in)).to(dt)
        S = ([3, 1], [0.625, 0.375])
        Wm, Wm_ex, _ = oracle.switch(W0, A, B, 1.5, None, S, with_stats=True, lib=lib)
        _, lhs, ab = oracle.gemv(Wm, x, with_stats=True, lib=lib)
        _, base, _ = oracle.gemv(W0, x, with_stats=True, lib=lib)
        _, ys, _ = oracle.sgmm(x.reshape(1, d_in), [S[0]], [S[1]], A, B, torch.zeros(1, d_out, dtype=dt), 1.5,
                               with_stats=True, lib=lib)
        rnd = (Wm.double() - Wm_ex).numpy() @ x.double().numpy()
        rhs = base.numpy() + ys.numpy()[0] + rnd
        assert np.allclose(lhs.numpy(), rhs, rtol=0, atol=1e-12 * (ab.numpy().max() + 1))


# ------------------------------------------------------------------ sgmm ----

def pin_sgmm_golden(lib):
    for c in _golden("sgmm_tiny.json")["cases"]:
        dt = torch.float32
        y = oracle.sgmm(_t(c["x"], dt), c["idx"], c["g"], _t(c["A"], dt), _t(c["B"], dt),
                        _t(c["y0"], dt), c["scale"], lib=lib)
        assert torch.equal(y, _t(c["y"], dt)), y


def pin_sgmm_gemm(lib):
    rng = _rng(31)
    E, r, d_in, d_out, T = 4, 3, 12, 7, 9
    for dt in (torch.float32, torch.bfloat16):
        A, B = _rand_bank(rng, E, r, d_in, d_out, dt)
        x = torch.from_numpy(rng.standard_normal((T, d_in))).to(dt)
        y0 = torch.from_numpy(rng.standard_normal((T, d_out))).to(dt)
        e0, e1, g0, g1 = 3, 1, 0.75, 0.25
        idx = torch.tensor([[e0, e1]] * T, dtype=torch.int32)
        g = torch.tensor([[g0, g1]] * T, dtype=torch.float32)
        _, ex, _ = oracle.sgmm(x, idx, g, A, B, y0, 1.5, with_stats=True, lib=lib)
        X, Ad, Bd = x.double().numpy(), A.double().numpy(), B.double().numpy()
        ref = y0.double().numpy() + 1.5 * (g0 * (X @ Ad[e0].T) @ Bd[e0].T + g1 * (X @ Ad[e1].T) @ Bd[e1].T)
        assert np.allclose(ex.numpy(), ref, rtol=1e-12, atol=1e-12)


def pin_sgmm_brute(lib):
    rng = _rng(32)
    for trial in range(10):
        E, r = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        d_in, d_out, T = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(1, 8))
        A, B = _rand_bank(rng, E, r, d_in, d_out, torch.float32)
        x = torch.from_numpy(rng.standard_normal((T, d_in))).float()
        y0 = torch.from_numpy(rng.standard_normal((T, d_out))).float()
        idx = rng.integers(-1, E, size=(T, 2)).astype(np.int32)
        g = rng.random((T, 2)).astype(np.float32)
        y, ex, ab = oracle.sgmm(x, idx, g, A, B, y0, 2.0, with_stats=True, lib=lib)
        ref = brute.sgmm(x, idx, g, A, B, y0, 2.0)
        assert np.allclose(ex.numpy(), ref, rtol=1e-12, atol=1e-12), (trial, ex, ref)
        assert torch.equal(y, torch.from_numpy(ref).float())
        assert (ab.numpy() + 1e-12 >= np.abs(ref)).all()


def pin_sgmm_absum(lib):
    """S of an SGMM output = |y| + sum_k |s g_k| * ((|x| @ |A_e|^T) @ |B_e|^T),
    equal both ways, for used, empty and duplicated slots."""
    rng = _rng(34)
    for trial in range(10):
        E, r = int(rng.integers(1, 5)), int(rng.integers(1, 6))
        d_in, d_out, T = int(rng.integers(1, 12)), int(rng.integers(1, 9)), int(rng.integers(1, 8))
        s = float(rng.choice([1.0, 2.0, -0.5]))
        for dt in (torch.float32, torch.bfloat16):
            A, B = _rand_bank(rng, E, r, d_in, d_out, dt)
            x = torch.from_numpy(rng.standard_normal((T, d_in))).to(dt)
            y0 = torch.from_numpy(rng.standard_normal((T, d_out))).to(dt)
            idx = rng.integers(-1, E, size=(T, 2)).astype(np.int32)
            g = (rng.random((T, 2)) - 0.25).astype(np.float32)
            _, _, ab = oracle.sgmm(x, idx, g, A, B, y0, s, with_stats=True, lib=lib)
            X, Ad, Bd = np.abs(x.double().numpy()), np.abs(A.double().numpy()), np.abs(B.double().numpy())
            ref = np.abs(y0.double().numpy()).copy()
            for t in range(T):
                for k in range(2):
                    e = idx[t, k]
                    if e >= 0:
                        ref[t] += abs(s * float(g[t, k])) * ((X[t] @ Ad[e].T) @ Bd[e].T)
            assert np.allclose(ab.numpy(), ref, rtol=1e-12, atol=0), (trial, ab, ref)


def pin_sgmm_properties(lib):
    rng = _rng(33)
    E, r, d_in, d_out, T = 4, 4, 16, 8, 12
    A, B = _rand_bank(rng, E, r, d_in, d_out, torch.bfloat16)
    x = torch.from_numpy(rng.standard_normal((T, d_in))).bfloat16()
    y0 = torch.from_numpy(rng.standard_normal((T, d_out))).bfloat16()
    idx = torch.from_numpy(rng.integers(0, E, size=(T, 2)).astype(np.int32))
    g = torch.from_numpy(rng.random((T, 2)).astype(np.float32))
    # zero gates leave y bitwise unchanged
    assert torch.equal(oracle.sgmm(x, idx, torch.zeros_like(g), A, B, y0, 1.0, lib=lib), y0)
    y = oracle.sgmm(x, idx, g, A, B, y0, 1.0, lib=lib)
    # slot order does not matter
    y_sw = oracle.sgmm(x, idx.flip(1).contiguous(), g.flip(1).contiguous(), A, B, y0, 1.0, lib=lib)
    assert torch.equal(y, y_sw)
    # rows are independent
    p = torch.from_numpy(rng.permutation(T))
    y_p = oracle.sgmm(x[p].contiguous(), idx[p].contiguous(), g[p].contiguous(), A, B,
                      y0[p].contiguous(), 1.0, lib=lib)
    assert torch.equal(y_p, y[p])
    # one expert, one slot: plain LoRA y + s*g*B(Ax)
    _, ex, _ = oracle.sgmm(x, torch.tensor([[0, -1]] * T, dtype=torch.int32),
                           torch.tensor([[1.0, 0.0]] * T), A[:1].contiguous(), B[:1].contiguous(),
                           y0, 2.0, with_stats=True, lib=lib)
    X, Ad, Bd = x.double().numpy(), A.double().numpy(), B.double().numpy()
    assert np.allclose(ex.numpy(), y0.double().numpy() + 2.0 * (X @ Ad[0].T) @ Bd[0].T, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- rounding ----

def pin_rounding(lib):
    cases = _golden("bf16_rounding.json")["cases"]
    v = np.array([c[0] for c in cases], np.float64)
    want = np.array([int(c[1], 16) for c in cases], np.uint16)
    got = oracle.round_to(v, 1, lib=lib)
    assert (got == want).all(), [(a, hex(b), hex(c)) for a, b, c in zip(v, got, want) if b != c]
    # fp32: the C conversion, checked against numpy's nearest-even cast
    rng = _rng(41)
    w = rng.standard_normal(1000) * 10.0 ** rng.integers(-40, 38, 1000)
    assert (oracle.round_to(w, 0, lib=lib) == w.astype(np.float32)).all()
    # bf16 on random values agrees with torch's nearest-even cast from binary64
    u = rng.standard_normal(5000) * 10.0 ** rng.integers(-38, 38, 5000)
    tb = torch.from_numpy(u).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.round_to(u, 1, lib=lib) == tb).all()


ALL_PINS = [
    pin_router_golden, pin_router_brute, pin_router_closed_form, pin_router_permutation,
    pin_router_bound,
    pin_switch_golden, pin_switch_premerge, pin_switch_general, pin_switch_absum, pin_switch_noop,
    pin_switch_roundtrip, pin_merged_equals_unmerged,
    pin_gemv_golden, pin_gemv_numpy, pin_gemv_merged,
    pin_centroid_golden, pin_centroid_brute, pin_centroid_invariants,
    pin_sgmm_golden, pin_sgmm_gemm, pin_sgmm_brute, pin_sgmm_absum, pin_sgmm_properties,
    pin_rounding,
]


def failing_pins(lib):
    """Names of the pins that fail (or crash) on a library handle."""
    bad = []
    for p in ALL_PINS:
        try:
            p(lib)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            bad.append(p.__name__)
    return bad
