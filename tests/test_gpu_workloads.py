"""Parity at the full workload sizes, in the launch configuration the benchmark
times (one switch launch over every adapted weight of every layer; one grouped
SGMM over every projection).  Outputs are sampled: the oracle recomputes the
sampled rows from the generated pre-state, row by row (each switched element
depends only on its own row of B and column of A; each SGMM row only on its own
x row), so the sample is an exact check of those outputs."""
import gc

import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth
from gpu_util import check_bf16, dev_set, host_set, sample_rows

pytestmark = pytest.mark.gpu

SPLIT = 2.0 ** -16


def _switch_sampled(wl, model, rows_per_w, old, new, what):
    rng = np.random.default_rng(7)
    pre = []
    for l, name, W, A, B in model:
        rows = sample_rows(W.shape[0], rows_per_w, rng)
        pre.append((rows, W[torch.from_numpy(rows).cuda()].cpu()))
    return pre


def _check_sampled(wl, model, pre, old, new, what):
    agg = {"n": 0, "n_gt2ulp": 0, "n_floor_only": 0, "max_ulp": 0}
    for (l, name, W, A, B), (rows, W0r) in zip(model, pre):
        got = W[torch.from_numpy(rows).cuda()].cpu()
        ref, ex, ab = oracle.switch_rows(W0r, rows, A.cpu(), B.cpu(), W.shape[0], wl.scale, old, new,
                                         with_stats=True)
        st = check_bf16(got, ref, ex, ab, 4 * wl.r + 2, what=f"{what} L{l}.{name}")
        for k in ("n", "n_gt2ulp", "n_floor_only"):
            agg[k] += st[k]
        agg["max_ulp"] = max(agg["max_ulp"], st["max_ulp"])
    print(what, agg, flush=True)
    return agg


def test_7b_decode_switch_sampled():
    wl = synth.WORKLOADS["7b-decode"]
    print("[workload] 7b-decode switch: building", flush=True)
    model = synth.switch_model(wl)
    x, Wr = synth.router_inputs(wl)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    idx, g = dlm.pregate(x, Wr)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), ri)
    W0 = [W.clone() for _, _, W, _, _ in model]
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    assert L.launches_per_switch() == 1
    steps = [0, 1, 2, 137, 255]
    for t in steps:
        old = None if t == 0 else host_set(ri[t - 1], rg[t - 1])
        new = host_set(ri[t], rg[t])
        for (_, _, W, _, _), w0 in zip(model, W0):
            W.copy_(w0)
        pre = _switch_sampled(wl, model, 3, old, new, "7b")
        if t == 137:
            # the decode loop's own form: the router's device output feeds the switch
            L.switch((idx[t - 1], g[t - 1]), (idx[t], g[t]))
        else:
            L.switch(dev_set(old), dev_set(new))
        torch.cuda.synchronize()
        print(f"[workload] 7b-decode step {t}", flush=True)
        _check_sampled(wl, model, pre, old, new, f"7b step {t}")
    assert L.status() == dlm.DLM_OK
    L.close()
    del model, W0
    gc.collect()
    torch.cuda.empty_cache()


def test_70b_decode_switch_sampled():
    wl = synth.WORKLOADS["70b-decode"]
    free, total = torch.cuda.mem_get_info()
    need = wl.switch_w_elems() * 2 * 1.25
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, have {free / 2**30:.0f}")
    print("[workload] 70b-decode switch: building", flush=True)
    model = synth.switch_model(wl)
    x, Wr = synth.router_inputs(wl)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    for t in (0, 64):
        old = None if t == 0 else host_set(ri[t - 1], rg[t - 1])
        new = host_set(ri[t], rg[t])
        if t > 0:
            synth.refill_switch_weights_(wl, model)   # back to the generated pre-state
        pre = _switch_sampled(wl, model, 2, old, new, "70b")
        L.switch(dev_set(old), dev_set(new))
        torch.cuda.synchronize()
        print(f"[workload] 70b-decode step {t}", flush=True)
        _check_sampled(wl, model, pre, old, new, f"70b step {t}")
    assert L.status() == dlm.DLM_OK
    L.close()
    del model
    gc.collect()
    torch.cuda.empty_cache()


def _sgmm_check_rows(wl, probs, ys, idx, g, rows, what):
    agg = {"n": 0, "n_gt2ulp": 0, "n_floor_only": 0, "max_ulp": 0}
    rt = torch.from_numpy(rows)
    for (l, name, x, A, B, y0), y in zip(probs, ys):
        xs, y0s = x[rt.cuda()].cpu(), y0[rt.cuda()].cpu()
        ref, ex, ab = oracle.sgmm(xs, idx[rt], g[rt], A.cpu(), B.cpu(), y0s, wl.scale,
                                  with_stats=True)
        st = check_bf16(y[rt.cuda()].cpu(), ref, ex, ab, x.shape[1] + 2 * wl.r + 2, extra=SPLIT,
                        what=f"{what} L{l}.{name}")
        for k in ("n", "n_gt2ulp", "n_floor_only"):
            agg[k] += st[k]
        agg["max_ulp"] = max(agg["max_ulp"], st["max_ulp"])
    print(what, agg, flush=True)


def test_sgmm_prefill_grouped_sampled():
    wl = synth.WORKLOADS["sgmm-prefill"]
    print("[workload] sgmm-prefill: building", flush=True)
    probs = synth.sgmm_problems(wl)
    idx, g = synth.batched_sets(wl)
    ys = [y0.clone() for *_, y0 in probs]
    grp = dlm.SgmmGroup([(x, A, B, y) for (_, _, x, A, B, _), y in zip(probs, ys)], wl.E, wl.r, wl.scale)
    ws = grp.run(idx.cuda(), g.cuda())
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(wl.T - 40, wl.T),
                                     rng.choice(wl.T, 160, replace=False)]))
    _sgmm_check_rows(wl, probs, ys, idx, g, rows, "prefill")
    grp.close()


def test_mixed_decode_grouped_sampled():
    wl = synth.WORKLOADS["mixed-decode"]
    print("[workload] mixed-decode: building", flush=True)
    probs = synth.sgmm_problems(wl)
    idx, g = synth.batched_sets(wl)
    ys = [y0.clone() for *_, y0 in probs]
    grp = dlm.SgmmGroup([(x, A, B, y) for (_, _, x, A, B, _), y in zip(probs, ys)], wl.E, wl.r, wl.scale)
    ws = grp.workspace(wl.T)
    rng = np.random.default_rng(4)
    for step in (0, 1, 77, 127):
        for y, (*_, y0) in zip(ys, probs):
            y.copy_(y0)
        grp.run(idx[step].cuda(), g[step].cuda(), workspace=ws)
        assert dlm.sgmm_status(ws) == dlm.DLM_OK
        print(f"[workload] mixed-decode step {step}", flush=True)
        rows = np.sort(rng.choice(wl.T, 8, replace=False))
        _sgmm_check_rows(wl, probs, ys, idx[step], g[step], rows, f"mixed step {step}")
    grp.close()


def test_7b_decode_fused_switch_and_product_per_layer_sampled():
    """The decode loop's fused form at its full size: one layer handle of the
    7B-shaped workload (7 projections), dlm_switch_gemv with the router's device
    sets.  Sampled rows of W' against the oracle's switch of those rows; the same
    rows of y against the oracle's product of those switched rows with x."""
    from test_gpu_gemv import _bf16_ulp, _check_y
    from gpu_util import gamma
    wl = synth.WORKLOADS["7b-decode"]
    print("[workload] 7b-decode fused switch + product: building one layer", flush=True)
    model = synth.switch_model(wl, layers=[5])
    x, Wr = synth.router_inputs(wl)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    idx, g = dlm.pregate(x, Wr)
    xs = [synth.normal_device((W.shape[1],), 1.0, wl.dtype, "cuda", wl.cfg_id, "xin", 5, k)
          for k, (_, _, W, _, _) in enumerate(model)]
    ys = [torch.full((W.shape[0],), float("nan"), dtype=torch.float32, device="cuda") for _, _, W, _, _ in model]
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    L.bind_vectors(xs, ys)
    W0 = [W.clone() for _, _, W, _, _ in model]
    for t in (0, 41):
        for (_, _, W, _, _), w0 in zip(model, W0):
            W.copy_(w0)
        old = None if t == 0 else host_set(ri[t - 1], rg[t - 1])
        new = host_set(ri[t], rg[t])
        pre = _switch_sampled(wl, model, 4, old, new, "7b fused")
        L.switch_gemv(None if t == 0 else (idx[t - 1], g[t - 1]), (idx[t], g[t]))
        torch.cuda.synchronize()
        print(f"[workload] 7b-decode fused step {t}", flush=True)
        _check_sampled(wl, model, pre, old, new, f"7b fused step {t}")
        for (l, name, W, A, B), (rows, W0r), xv, y in zip(model, pre, xs, ys):
            ref, ex, ab = oracle.switch_rows(W0r, rows, A.cpu(), B.cpu(), W.shape[0], wl.scale, old, new,
                                             with_stats=True)
            wtol = np.maximum(2 * _bf16_ulp(ref.double().numpy()), gamma(4 * wl.r + 2) * ab.numpy())
            _check_y(y[torch.from_numpy(rows).cuda()], ref, wtol, xv, f"7b fused step {t} {name}")
    assert L.status() == dlm.DLM_OK
    L.close()
    del model, W0
    gc.collect()
    torch.cuda.empty_cache()


def test_70b_decode_switch_and_product_per_layer_sampled():
    """dlm_switch_gemv on one layer of the 70B-shaped workload (rank 64: the wide
    switch, then the product kernel; d_in up to 28672). Sampled rows of W' and y
    against the oracle, as in the 7B-shaped fused test."""
    from test_gpu_gemv import _bf16_ulp, _check_y
    from gpu_util import gamma
    wl = synth.WORKLOADS["70b-decode"]
    print("[workload] 70b-decode switch + product: building one layer", flush=True)
    model = synth.switch_model(wl, layers=[11])
    x, Wr = synth.router_inputs(wl)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    idx, g = dlm.pregate(x, Wr)
    xs = [synth.normal_device((W.shape[1],), 1.0, wl.dtype, "cuda", wl.cfg_id, "xin", 11, k)
          for k, (_, _, W, _, _) in enumerate(model)]
    ys = [torch.full((W.shape[0],), float("nan"), dtype=torch.float32, device="cuda") for _, _, W, _, _ in model]
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    L.bind_vectors(xs, ys)
    t = 9
    old, new = host_set(ri[t - 1], rg[t - 1]), host_set(ri[t], rg[t])
    pre = _switch_sampled(wl, model, 4, old, new, "70b product")
    L.switch_gemv((idx[t - 1], g[t - 1]), (idx[t], g[t]))
    torch.cuda.synchronize()
    print("[workload] 70b-decode switch + product: checking", flush=True)
    _check_sampled(wl, model, pre, old, new, "70b product")
    for (l, name, W, A, B), (rows, W0r), xv, y in zip(model, pre, xs, ys):
        ref, ex, ab = oracle.switch_rows(W0r, rows, A.cpu(), B.cpu(), W.shape[0], wl.scale, old, new,
                                         with_stats=True)
        wtol = np.maximum(2 * _bf16_ulp(ref.double().numpy()), gamma(4 * wl.r + 2) * ab.numpy())
        _check_y(y[torch.from_numpy(rows).cuda()], ref, wtol, xv, f"70b product {name}")
    assert L.status() == dlm.DLM_OK
    L.close()
    del model
    gc.collect()
    torch.cuda.empty_cache()
