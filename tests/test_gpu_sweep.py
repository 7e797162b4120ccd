"""Seeded sweeps of random valid shapes for the fused switch and the SGMM,
each compared element by element with the oracle (same checks and tolerances
as the hand-picked cases). The generator draws every size class the kernels
distinguish: ragged rows and columns, ranks below, at and between multiples of
16 (and not multiples of 8), one to 32 experts, bf16 and fp32, K beyond one
SGMM slice, empty and duplicated slots."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
from gpu_util import dev_set
from test_gpu_sgmm import _check, _problem, _sets
from test_gpu_switch import _compare, _model

pytestmark = pytest.mark.gpu

N_SWITCH = 48
N_SGMM = 48


def _rank(rng):
    return int(rng.choice([1, 3, 8, 12, 16, 17, 24, 31, 32, 40, 48, 56, 64, 72, 88, 100, 120, 128]))


def _switch_config(i):
    rng = np.random.default_rng(70000 + i)
    dt = torch.float32 if rng.random() < 0.15 else torch.bfloat16
    n = int(rng.integers(1, 4))
    shapes = []
    for _ in range(n):
        d_out = int(rng.integers(1, 600))
        d_in = 8 * int(rng.integers(1, 160))
        shapes.append((d_out, d_in))
    E = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    return shapes, E, _rank(rng), float(rng.choice([0.5, 1.0, 2.0])), dt


def _sgmm_config(i):
    rng = np.random.default_rng(80000 + i)
    dt = torch.float32 if rng.random() < 0.15 else torch.bfloat16
    T = int(rng.integers(1, 700))
    d_in = 8 * int(rng.integers(1, 220))
    d_out = 8 * int(rng.integers(1, 90))
    E = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    return T, d_in, d_out, E, _rank(rng), float(rng.choice([0.5, 1.0, 2.0])), dt


@pytest.mark.parametrize("i", range(N_SWITCH))
def test_switch_sweep(i):
    shapes, E, r, scale, dt = _switch_config(i)
    print(f"[sweep switch {i}] shapes={shapes} E={E} r={r} scale={scale} {dt}", flush=True)
    model = _model(shapes, E, r, dt, 71000 + i)
    W0s = [W.cpu().clone() for W, _, _ in model]
    rng = np.random.default_rng(72000 + i)
    L = dlm.Layers(model, E, r, scale)

    def a_set():
        e = rng.choice(E, size=2, replace=E < 2).tolist()
        if rng.random() < 0.2:
            e[1] = -1
        g = rng.random(2).astype(np.float32).tolist()
        return e, g

    prev = None
    for k in range(3):
        new = a_set()
        for (W, _, _), W0 in zip(model, W0s):
            W.copy_(W0)
        L.switch(dev_set(prev), dev_set(new))
        torch.cuda.synchronize()
        _compare(model, W0s, scale, prev, new, f"sweep{i} step{k}", dt)
        prev = new
    assert L.status() == dlm.DLM_OK
    L.close()


@pytest.mark.parametrize("i", range(N_SGMM))
def test_sgmm_sweep(i):
    T, d_in, d_out, E, r, scale, dt = _sgmm_config(i)
    print(f"[sweep sgmm {i}] T={T} d_in={d_in} d_out={d_out} E={E} r={r} scale={scale} {dt}", flush=True)
    x, A, B, y = _problem(T, d_in, d_out, E, r, dt, 81000 + i)
    idx, g = _sets(T, E, np.random.default_rng(82000 + i))
    y0 = y.cpu().clone()
    ws = dlm.sgmm_workspace(T, d_in, E, r)
    dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y, scale, ws)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    _check(x, idx, g, A, B, y0, y, scale, f"sgmm sweep {i}")
    none = (idx == -1).all(1)
    assert torch.equal(y.cpu()[none], y0[none])


N_SGMM_WIDE = 8


@pytest.mark.parametrize("i", range(N_SGMM_WIDE))
def test_sgmm_sweep_several_k_slices(i):
    """Random shapes with d_in past one 2048-wide K slice (2 to 5 slices), every
    rank class: the expand adds the slices' partials itself up to rank 64, a
    K-slice sum launch does it above."""
    rng = np.random.default_rng(83000 + i)
    T = int(rng.integers(1, 300))
    d_in = 8 * int(rng.integers(257, 1250))
    d_out = 8 * int(rng.integers(1, 60))
    E = int(rng.choice([1, 2, 4, 8, 16]))
    r = _rank(rng)
    scale = float(rng.choice([0.5, 1.0, 2.0]))
    print(f"[sweep sgmm wide {i}] T={T} d_in={d_in} d_out={d_out} E={E} r={r} scale={scale}", flush=True)
    x, A, B, y = _problem(T, d_in, d_out, E, r, torch.bfloat16, 84000 + i)
    idx, g = _sets(T, E, np.random.default_rng(85000 + i))
    y0 = y.cpu().clone()
    ws = dlm.sgmm_workspace(T, d_in, E, r)
    dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y, scale, ws)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    _check(x, idx, g, A, B, y0, y, scale, f"sgmm wide sweep {i}")


N_ROUTER = 24
N_PRODUCT = 20


def _router_config(i):
    rng = np.random.default_rng(90000 + i)
    dt = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    d = int(rng.choice([1, 7, 64, 100, 520, 1000, 4096, 8192])) if rng.random() < 0.5 else 8 * int(rng.integers(1, 700))
    return int(rng.integers(1, 300)), d, dt, rng


@pytest.mark.parametrize("i", range(N_ROUTER))
def test_router_sweep(i):
    from test_gpu_pregate import _check, _xw
    T, d, dt, rng = _router_config(i)
    E = int(rng.integers(2, 33))
    x, Wr = _xw(T, d, E, dt, 91000 + i)
    _check(x, Wr, f"sweep {i}")


@pytest.mark.parametrize("i", range(N_ROUTER))
def test_centroid_router_sweep(i):
    from test_gpu_pregate import _check_centroid, _xc
    T, d, dt, rng = _router_config(100 + i)
    E, J = int(rng.integers(1, 33)), int(rng.choice([1, 2, 3, 4, 9, 16]))
    x, C = _xc(T, d, E, J, dt, 92000 + i)
    _check_centroid(x, C, f"sweep {i} E={E} J={J}")


@pytest.mark.parametrize("i", range(N_PRODUCT))
def test_switch_gemv_sweep(i):
    """dlm_switch_gemv on random shapes: W' bitwise equal to a plain dlm_switch of
    a twin, y against the oracle's product with the oracle's switched weights."""
    from test_gpu_gemv import _bf16_ulp, _check_y, _vectors
    import oracle
    from gpu_util import check_bf16, check_f32, gamma
    shapes, E, r, scale, dt = _switch_config(200 + i)
    if i % 2 == 0:
        r = int(np.random.default_rng(93000 + i).choice([1, 4, 8, 16]))  # the fused kernel's ranks
    print(f"[sweep switch_gemv {i}] shapes={shapes} E={E} r={r} scale={scale} {dt}", flush=True)
    model = _model(shapes, E, r, dt, 94000 + i)
    twin = [(W.clone(), A, B) for W, A, B in model]
    W0s = [W.cpu().clone() for W, _, _ in model]
    xs, ys = _vectors(shapes, dt, 94000 + i)
    L = dlm.Layers(model, E, r, scale)
    L.bind_vectors(xs, ys)
    Tw = dlm.Layers(twin, E, r, scale)
    rng = np.random.default_rng(95000 + i)
    old = (rng.choice(E, size=2, replace=E < 2).tolist(), rng.random(2).astype(np.float32).tolist())
    new = (rng.choice(E, size=2, replace=E < 2).tolist(), rng.random(2).astype(np.float32).tolist())
    L.switch_gemv(dev_set(old), dev_set(new))
    Tw.switch(dev_set(old), dev_set(new))
    torch.cuda.synchronize()
    for k, ((W, A, B), (Wt, _, _), w0, x, y) in enumerate(zip(model, twin, W0s, xs, ys)):
        assert torch.equal(W, Wt), f"sweep {i} w{k}: fused switch differs from dlm_switch"
        ref, ex, ab = oracle.switch(w0, A.cpu(), B.cpu(), scale, old, new, with_stats=True)
        if dt == torch.bfloat16:
            check_bf16(W.cpu(), ref, ex, ab, 4 * r + 2, what=f"sweep {i} w{k}")
            wtol = np.maximum(2 * _bf16_ulp(ref.double().numpy()), gamma(4 * r + 2) * ab.numpy())
        else:
            check_f32(W.cpu(), ex, ab, 4 * r + 2, f"sweep {i} w{k}")
            wtol = np.maximum(1e-5 * np.abs(ex.numpy()), gamma(4 * r + 2) * ab.numpy())
        _check_y(y, ref, wtol, x, f"sweep {i} w{k}")
    assert L.status() == dlm.DLM_OK
    L.close()
    Tw.close()


N_GROUP = 16


@pytest.mark.parametrize("i", range(N_GROUP))
def test_sgmm_group_sweep(i):
    """Random groups of 2-7 problems with their own d_in / d_out (some sharing an
    A/B bank) run on one segmentation; every problem's y against the oracle."""
    rng = np.random.default_rng(96000 + i)
    dt = torch.float32 if i % 5 == 4 else torch.bfloat16
    T = int(rng.integers(1, 500))
    E = int(rng.choice([1, 2, 4, 8, 16, 32]))
    r = _rank(rng)
    scale = float(rng.choice([0.5, 1.0, 2.0]))
    n = int(rng.integers(2, 8))
    probs, banks = [], []
    for k in range(n):
        if banks and rng.random() < 0.3:
            d_in, d_out, A, B = banks[int(rng.integers(len(banks)))]   # a shared bank
        else:
            d_in, d_out = 8 * int(rng.integers(1, 200)), 8 * int(rng.integers(1, 80))
            _, A, B, _ = _problem(1, d_in, d_out, E, r, dt, (97000 + i, k))
            banks.append((d_in, d_out, A, B))
        x, _, _, y = _problem(T, d_in, d_out, 1, 1, dt, (98000 + i, k))
        probs.append((x, A, B, y))
    print(f"[sweep group {i}] T={T} E={E} r={r} {dt} problems={[(p[0].shape[1], p[3].shape[1]) for p in probs]}",
          flush=True)
    idx, g = _sets(T, E, np.random.default_rng(99000 + i))
    y0s = [y.cpu().clone() for *_, y in probs]
    grp = dlm.SgmmGroup(probs, E, r, scale)
    ws = grp.run(idx.cuda(), g.cuda())
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    for k, ((x, A, B, y), y0) in enumerate(zip(probs, y0s)):
        _check(x, idx, g, A, B, y0, y, scale, f"group sweep {i} problem {k}")
    grp.close()


N_UNMERGED = 24


def _unmerged_config(i):
    rng = np.random.default_rng(96000 + i)
    dt = torch.float32 if rng.random() < 0.2 else torch.bfloat16
    shapes = []
    for _ in range(int(rng.integers(1, 5))):
        d_out = int(rng.integers(1, 600))
        d_in = 8 * int(rng.integers(1, 1600 if rng.random() < 0.5 else 160))  # up to 7 K slices
        shapes.append((d_out, d_in))
    E = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    e = rng.choice(E, size=2, replace=E < 2).tolist()
    if rng.random() < 0.2:
        e[int(rng.integers(0, 2))] = -1
    g = rng.random(2).astype(np.float32).tolist()
    return shapes, E, _rank(rng), float(rng.choice([0.5, 1.0, 2.0])), dt, (e, g)


@pytest.mark.parametrize("i", range(N_UNMERGED))
def test_gemv_unmerged_sweep(i):
    """dlm_gemv_unmerged on random shapes and sets: y against the oracle's
    product plus its unmerged adapters (the hand-picked cases' bound), W
    untouched."""
    from test_gpu_unmerged import _check, _model as _um_model, _vectors as _um_vectors
    shapes, E, r, scale, dt, s = _unmerged_config(i)
    print(f"[sweep unmerged {i}] shapes={shapes} E={E} r={r} scale={scale} {dt} set={s}", flush=True)
    model = _um_model(shapes, E, r, dt, 97000 + i)
    W0 = [W.clone() for W, _, _ in model]
    xs, ys = _um_vectors(shapes, dt, 97000 + i)
    L = dlm.Layers(model, E, r, scale)
    L.bind_vectors(xs, ys)
    L.gemv_unmerged(dev_set(s))
    assert L.status() == dlm.DLM_OK
    _check(model, xs, ys, s, E, r, scale, f"sweep unmerged {i}")
    assert all(torch.equal(W, w0) for (W, _, _), w0 in zip(model, W0))
    L.close()
