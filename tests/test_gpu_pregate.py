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


# ---- nearest-centroid pre-gate ------------------------------------------------

def _check_centroid(x, C, what):
    """Slot 0 bit-exact wherever the nearest adapter is farther from a tie than
    twice the binary64 summation bound of its distance; near ties the GPU's pick
    must be within that bound of the oracle's.  Slot 1 empty, g = (1, 0)."""
    print(f"[centroid] {what} T={x.shape[0]} d={x.shape[1]} E={C.shape[0]} J={C.shape[1]} {x.dtype}", flush=True)
    idx, g = dlm.pregate_centroid(x, C)
    torch.cuda.synchronize()
    idx, g = idx.cpu(), g.cpu()
    ri, rg, dist, mg = oracle.pregate_centroid(x.cpu(), C.cpu(), with_stats=True)
    E = C.shape[0]
    assert (idx[:, 1] == -1).all() and (g[:, 0] == 1).all() and (g[:, 1] == 0).all()
    assert ((idx[:, 0] >= 0) & (idx[:, 0] < E)).all()
    d = x.shape[1]
    u = 2.0 ** -53
    bd = (d + 2) * u / (1 - (d + 2) * u) * dist.max(1).values.numpy()
    safe = mg.numpy() > 2 * bd
    assert (idx[:, 0].numpy()[safe] == ri[:, 0].numpy()[safe]).all(), f"{what}: centroid index mismatch"
    dd = dist.numpy()
    for t in np.nonzero(~safe)[0]:
        assert dd[t, idx[t, 0]] - dd[t, ri[t, 0]] <= 2 * bd[t], (what, t)
    return int((~safe).sum())


def _xc(T, d, E, J, dt, *keys):
    x = synth.normal_device((T, d), 1.0, dt, "cuda", *keys, "x")
    C = synth.normal_device((E, J, d), 1.0, dt, "cuda", *keys, "C")
    return x, C


@pytest.mark.parametrize("T,d,E,J,dt", [(16, 64, 4, 2, torch.float32), (256, 4096, 8, 4, torch.bfloat16),
                                        (128, 8192, 16, 2, torch.bfloat16), (37, 100, 3, 5, torch.bfloat16),
                                        (5, 1, 1, 1, torch.float32), (64, 256, 32, 3, torch.bfloat16),
                                        (1, 4096, 8, 1, torch.bfloat16), (9, 520, 7, 9, torch.float32)])
def test_centroid_router_shapes(T, d, E, J, dt):
    x, C = _xc(T, d, E, J, dt, 4000, T, d, E, J)
    assert _check_centroid(x, C, f"shape {T}x{d} E={E} J={J}") == 0


def test_centroid_router_ties_and_exact_hits():
    d, E, J = 96, 6, 3
    x, C = _xc(5, d, E, J, torch.bfloat16, 4100)
    C[4] = C[1]                 # a duplicated adapter never beats its lower-indexed twin
    x[0] = C[3, 2]              # a token on a centroid picks its adapter (distance 0)
    x[1] = C[1, 0]              # ... and on a duplicated one, the lower index
    idx, g = dlm.pregate_centroid(x, C)
    torch.cuda.synchronize()
    assert idx[0, 0].item() == 3 and idx[1, 0].item() == 1
    assert (idx[:, 0] != 4).all()
    _check_centroid(x, C, "ties")


def test_centroid_router_feeds_the_switch():
    """The centroid router's one-slot sets drive the fused switch directly."""
    E, r, d = 6, 16, 256
    x, C = _xc(2, d, E, 2, torch.bfloat16, 4200)
    W = synth.normal_device((128, d), 0.02, torch.bfloat16, "cuda", 4200, "W")
    A = synth.normal_device((E, r, d), 0.02, torch.bfloat16, "cuda", 4200, "A")
    B = synth.normal_device((E, 128, r), 0.02, torch.bfloat16, "cuda", 4200, "B")
    W0 = W.cpu().clone()
    idx, g = dlm.pregate_centroid(x, C)
    L = dlm.Layers([(W, A, B)], E, r, 1.0)
    L.switch((idx[0], g[0]), (idx[1], g[1]))
    torch.cuda.synchronize()
    ri, rg = oracle.pregate_centroid(x.cpu(), C.cpu())
    assert torch.equal(ri, idx.cpu())
    from gpu_util import check_bf16, host_set
    ref, ex, ab = oracle.switch(W0, A.cpu(), B.cpu(), 1.0, host_set(ri[0], rg[0]), host_set(ri[1], rg[1]),
                                with_stats=True)
    check_bf16(W.cpu(), ref, ex, ab, 4 * r + 2, what="centroid->switch")
    assert L.status() == dlm.DLM_OK
    L.close()


def test_centroid_router_empty_batch_is_noop():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(4, 2, 64, dtype=torch.bfloat16, device="cuda")
    idx, g = dlm.pregate_centroid(x, C)
    assert idx.shape == (0, 2)


def _scan_top2(l):
    """Strict '>' scans from the lowest candidate index, as the oracle's."""
    i0 = 0
    for e in range(1, len(l)):
        if l[e] > l[i0]:
            i0 = e
    i1 = 1 if i0 == 0 else 0
    for e in range(len(l)):
        if e != i0 and l[e] > l[i1]:
            i1 = e
    return [i0, i1]


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("E", [2, 3, 8, 17, 32])
def test_router_top2_on_crafted_logits(E, dt):
    """The wavefront top two on logit vectors set exactly (one token, x a unit
    vector, Wr's first row the logits): NaN where slot 0's scan starts, where
    slot 1's starts and elsewhere, infinities, many-way ties.  Indices are
    bit-exact against the oracle's scans (bf16 with E a multiple of 8 takes the
    vectorised kernel, the rest the one-wave kernel); weights are compared on
    the finite vectors."""
    nan, inf = float("nan"), float("inf")
    fixed = [[nan] + [1.0] * (E - 1), [1.0, nan] + [2.0] * (E - 2), [5.0, nan] + [3.0] * (E - 2),
             [-inf] * E, [inf] * E, [0.5] * E, [nan] * E, [1.0] * (E - 1) + [nan],
             [2.0, 2.0] + [nan] * (E - 2), [-inf, nan] + [-inf] * (E - 2), [0.0] * (E - 1) + [inf],
             [-1.0] * (E - 2) + [0.5, 0.5]]
    rng = np.random.default_rng(1000 + E)
    pool = np.array([nan, inf, -inf, -1.0, 0.0, 0.5, 1.0, 2.0])
    cases = [v[:E] for v in fixed] + [list(rng.choice(pool, size=E, p=[.1, .05, .1, .15, .15, .15, .15, .15]))
                                      for _ in range(40)]
    d = 8
    x = torch.zeros(1, d, dtype=dt)
    x[0, 0] = 1.0
    print(f"[pregate] crafted logits E={E} {dt}: {len(cases)} vectors", flush=True)
    for c, lv in enumerate(cases):
        Wr = torch.zeros(d, E, dtype=dt)
        Wr[0] = torch.tensor(lv, dtype=torch.float64).to(dt)
        idx, g = dlm.pregate(x.cuda(), Wr.cuda())
        torch.cuda.synchronize()
        ri, rg = oracle.pregate(x, Wr)
        got = idx[0].cpu().tolist()
        assert got == ri[0].tolist() == _scan_top2(Wr[0].double().tolist()), (c, lv, got, ri[0].tolist())
        if all(np.isfinite(lv)):
            gg, rr = g[0].cpu(), rg[0]
            assert ((gg - rr).abs() / rr.abs().clamp_min(1e-30)).max().item() <= 2.0 ** -22, (c, lv, gg, rr)
