"""Router (pre-gate) parity: HIP kernel vs the binary64 oracle.

Indices must be bit-exact wherever the decision is farther from a tie than the
binary64 summation bound (both sides sum in binary64, in different orders);
within that bound both choices are correct and the GPU's is checked to be one of
them.  Weights agree within 1 fp32 ulp (rel <= 1.2e-7), well inside rel 1e-5."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth

pytestmark = pytest.mark.gpu


def _check(x, Wr, what):
    print(f"[pregate] {what} T={x.shape[0]} d={x.shape[1]} E={Wr.shape[1]} {x.dtype}", flush=True)
    idx, g = dlm.pregate(x, Wr)
    torch.cuda.synchronize()
    idx, g = idx.cpu(), g.cpu()
    ri, rg, lg, mg, bd = oracle.pregate(x.cpu(), Wr.cpu(), with_stats=True)
    T, E = lg.shape
    assert ((idx >= 0) & (idx < E)).all() and (idx[:, 0] != idx[:, 1]).all()
    safe = (mg > 2 * bd).numpy()
    near = int((~safe).sum())
    assert (idx.numpy()[safe] == ri.numpy()[safe]).all(), f"{what}: router index mismatch"
    l = lg.numpy()
    for t in np.nonzero(~safe)[0]:
        # near-tie: the GPU's pick must be within the bound of the oracle's logits
        for k in range(2):
            assert abs(l[t, idx[t, k]] - l[t, ri[t, k]]) <= 2 * bd[t].item() + 0.0, (what, t)
    eq = torch.from_numpy((idx.numpy() == ri.numpy()).all(1))
    if eq.any():
        rel = (g[eq] - rg[eq]).abs() / rg[eq].abs().clamp_min(1e-30)
        assert rel.max().item() <= 2.0 ** -22, f"{what}: g rel {rel.max()}"
    return near


def _xw(T, d, E, dt, *keys):
    x = synth.normal_device((T, d), 1.0, dt, "cuda", *keys, "x")
    Wr = synth.normal_device((d, E), 0.02, dt, "cuda", *keys, "Wr")
    return x, Wr


@pytest.mark.parametrize("name", ["tiny-fp32", "7b-decode", "70b-decode"])
def test_workload_router(name):
    wl = synth.WORKLOADS[name]
    x, Wr = _xw(wl.T, wl.d_model, wl.E, wl.dtype, wl.cfg_id)
    assert _check(x, Wr, name) == 0


@pytest.mark.parametrize("name", ["sgmm-prefill", "mixed-decode"])
def test_router_on_batched_workload_shapes(name):
    # the batched workloads give their sets directly; the router is still checked at
    # their (d, E) with 256 tokens
    wl = synth.WORKLOADS[name]
    x, Wr = _xw(256, wl.d_model, wl.E, wl.dtype, wl.cfg_id, "router")
    assert _check(x, Wr, name) == 0


@pytest.mark.parametrize("T,d,E,dt", [(1, 4096, 8, torch.bfloat16), (3, 100, 2, torch.bfloat16),
                                      (65, 130, 32, torch.float32), (7, 64, 17, torch.bfloat16),
                                      (200, 1, 5, torch.float32), (5, 1000, 16, torch.bfloat16),
                                      (9, 520, 32, torch.bfloat16), (33, 8192, 24, torch.bfloat16)])
def test_router_shapes(T, d, E, dt):
    x, Wr = _xw(T, d, E, dt, 99, T, d, E)
    _check(x, Wr, f"shape {T}x{d}x{E}")


def test_router_ties_and_zero_input():
    d, E = 96, 8
    x = torch.zeros(4, d, dtype=torch.bfloat16, device="cuda")
    x[1:] = synth.normal_device((3, d), 1.0, torch.bfloat16, "cuda", 7, "x")
    Wr = synth.normal_device((d, E), 0.02, torch.bfloat16, "cuda", 7, "Wr")
    Wr[:, 5] = Wr[:, 2]       # exact duplicate: equal logits, lower index wins
    Wr[:, 6] = Wr[:, 2]
    idx, g = dlm.pregate(x, Wr)
    torch.cuda.synchronize()
    assert idx[0].tolist() == [0, 1] and g[0].tolist() == [0.5, 0.5]
    for t in range(1, 4):
        p = idx[t].tolist()
        assert 5 not in p or p == [2, 5]
        assert 6 not in p
    _check(x, Wr, "ties")


def test_router_non_finite_input_stays_in_range():
    x = torch.full((2, 64), float("nan"), dtype=torch.float32, device="cuda")
    Wr = torch.ones(64, 4, dtype=torch.float32, device="cuda")
    idx, _ = dlm.pregate(x, Wr)
    torch.cuda.synchronize()
    assert ((idx >= 0) & (idx < 4)).all() and (idx[:, 0] != idx[:, 1]).all()


def test_router_empty_batch_is_noop():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    Wr = torch.zeros(64, 8, dtype=torch.bfloat16, device="cuda")
    idx, g = dlm.pregate(x, Wr)
    assert idx.shape == (0, 2)
