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

N_SWITCH = 24
N_SGMM = 24


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
