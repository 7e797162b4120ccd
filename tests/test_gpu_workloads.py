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
from gpu_util import check_bf16, check_f32, dev_set, host_set, sample_rows

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
        n_terms = x.shape[1] + 2 * wl.r + 2
        if y.dtype == torch.float32:
            check_f32(y[rt.cuda()].cpu(), ex, ab, n_terms, what=f"{what} L{l}.{name}")
            continue
        st = check_bf16(y[rt.cuda()].cpu(), ref, ex, ab, n_terms, extra=SPLIT,
                        what=f"{what} L{l}.{name}")
        for k in ("n", "n_gt2ulp", "n_floor_only"):
            agg[k] += st[k]
        agg["max_ulp"] = max(agg["max_ulp"], st["max_ulp"])
    print(what, agg, flush=True)


@pytest.mark.parametrize("name,layer", [("tiny-fp32", 1), ("7b-decode", 3), ("70b-decode", 7)])
def test_sgmm_on_router_sets_every_row(name, layer):
    """The unmerged batched form on the decode workloads' own router sets: one
    layer's projections (7B-shaped: d up to 11008; 70B-shaped: rank 64, 16
    experts, d_in up to 28672) as one group over all the workload's tokens
    (16 / 256 / 128 rows), the router's device output feeding the SGMM.  Every
    row of every projection is checked against the oracle."""
    wl = synth.WORKLOADS[name]
    print(f"[workload] {name} SGMM on router sets: building layer {layer}", flush=True)
    x, Wr = synth.router_inputs(wl)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    idx, g = dlm.pregate(x, Wr)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), ri)
    probs = synth.sgmm_problems(wl, layers=[layer])
    ys = [y0.clone() for *_, y0 in probs]
    grp = dlm.SgmmGroup([(xp, A, B, y) for (_, _, xp, A, B, _), y in zip(probs, ys)], wl.E, wl.r, wl.scale)
    ws = grp.run(idx, g)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    print(f"[workload] {name} SGMM on router sets: checking", flush=True)
    _sgmm_check_rows(wl, probs, ys, ri, rg, np.arange(wl.T), f"{name} router-set SGMM")
    grp.close()
    del probs, ys
    gc.collect()
    torch.cuda.empty_cache()


def test_7b_decode_switch_full_layer_every_element():
    """One switch launch over all 32 layers of the 7B-shaped workload (the
    benchmark's launch), then one whole layer -- all 7 projections, every row
    and column, 202 M weights -- against the oracle element by element."""
    wl = synth.WORKLOADS["7b-decode"]
    print("[workload] 7b-decode full layer: building", flush=True)
    model = synth.switch_model(wl)
    x, Wr = synth.router_inputs(wl)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    idx, g = dlm.pregate(x, Wr)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), ri)
    layer, t = 17, 200
    mine = [(k, m) for k, m in enumerate(model) if m[0] == layer]
    W0 = {k: W.cpu() for k, (_, _, W, _, _) in mine}
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    L.switch((idx[t - 1], g[t - 1]), (idx[t], g[t]))
    torch.cuda.synchronize()
    assert L.status() == dlm.DLM_OK
    L.close()
    old, new = host_set(ri[t - 1], rg[t - 1]), host_set(ri[t], rg[t])
    agg = {"n": 0, "n_gt2ulp": 0, "n_floor_only": 0, "max_ulp": 0}
    for k, (l, name, W, A, B) in mine:
        print(f"[workload] 7b-decode full layer: checking {name}", flush=True)
        rows = np.arange(W.shape[0], dtype=np.int64)
        ref, ex, ab = oracle.switch_rows(W0[k], rows, A.cpu(), B.cpu(), W.shape[0], wl.scale, old, new,
                                         with_stats=True)
        st = check_bf16(W.cpu(), ref, ex, ab, 4 * wl.r + 2, what=f"7b full layer L{l}.{name}")
        for key in ("n", "n_gt2ulp", "n_floor_only"):
            agg[key] += st[key]
        agg["max_ulp"] = max(agg["max_ulp"], st["max_ulp"])
        del ref, ex, ab
    print("7b full layer", agg, flush=True)
    assert agg["n"] == sum(o * i for _, o, i in wl.projs)
    del model
    gc.collect()
    torch.cuda.empty_cache()


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


def test_mixed_decode_released_rows_full_step():
    """Rows that release their adapters (both slots empty) at the mixed decode
    workload's full size: all 224 projections (32 layers x 7) as one group of 64
    rows on one workspace, three steps in a row -- every row live, then the upper
    half released, then every third row released and every fifth live row with
    one slot only.  The live rows of every projection match the oracle element
    by element; every released row of y is left bitwise as it was."""
    wl = synth.WORKLOADS["mixed-decode"]
    print("[workload] mixed-decode released rows: building", flush=True)
    probs = synth.sgmm_problems(wl)
    idx, g = synth.batched_sets(wl)
    ys = [y0.clone() for *_, y0 in probs]
    grp = dlm.SgmmGroup([(x, A, B, y) for (_, _, x, A, B, _), y in zip(probs, ys)], wl.E, wl.r, wl.scale)
    ws = grp.workspace(wl.T)
    rows = np.arange(wl.T)
    cases = []
    i0, g0 = idx[5].clone(), g[5].clone()
    cases.append(("all live", i0, g0))
    i1, g1 = idx[6].clone(), g[6].clone()
    i1[wl.T // 2:], g1[wl.T // 2:] = -1, 0.0
    cases.append(("upper half released", i1, g1))
    i2, g2 = idx[7].clone(), g[7].clone()
    i2[0::3], g2[0::3] = -1, 0.0
    one = np.setdiff1d(np.arange(1, wl.T, 5), np.arange(0, wl.T, 3))
    i2[one, 1], g2[one, 1] = -1, 0.0
    cases.append(("every third released", i2, g2))
    for what, ic, gc_ in cases:
        for y, (*_, y0) in zip(ys, probs):
            y.copy_(y0)
        grp.run(ic.cuda(), gc_.cuda(), workspace=ws)
        assert dlm.sgmm_status(ws) == dlm.DLM_OK
        torch.cuda.synchronize()
        released = (ic == -1).all(1).numpy()
        print(f"[workload] mixed-decode {what}: {int(released.sum())} released rows, checking", flush=True)
        rel = torch.from_numpy(np.nonzero(released)[0]).cuda()
        for (l, name, *_, y0), y in zip(probs, ys):
            assert torch.equal(y[rel], y0[rel]), f"{what}: released rows of L{l}.{name} changed"
        _sgmm_check_rows(wl, probs, ys, ic, gc_, rows[~released], f"mixed {what}")
    grp.close()
    del probs, ys
    gc.collect()
    torch.cuda.empty_cache()


def _layerwise_outputs(lw):
    return ([t.clone() for t in lw.idx], [t.clone() for t in lw.g],
            [[y.clone() for y in yl] for yl in lw.y_lora], [[y.clone() for y in yl] for yl in lw.y_base])


def test_7b_layerwise_decode_token():
    """The layer-wise baseline (per-layer routing, unmerged adapters) at the
    7B-shaped workload's full size, 32 layers x 7 projections, one SGMM call per
    projection: one token eagerly, checked against the oracle -- every layer's
    router set (indices bit-exact), every projection's adapter output (T = 1,
    from zero) element by element, the base products of layers 0 and 31 element
    by element -- then the same token replayed three times from one HIP graph,
    each replay bitwise equal to the eager token.  Then the pre-gated unmerged
    form on the same layers (one router per token, one grouped SGMM per layer):
    every adapter output against the oracle with the first layer's set.  Last
    the fused unmerged form (one router per token, one dlm_gemv_unmerged per
    layer): layers 0, 15 and 31 against the oracle's product plus its unmerged
    adapters, every layer's output bitwise equal across two graph replays."""
    from dynamic_lora_moe_amd.layerwise import LayerwiseDecode
    wl = synth.WORKLOADS["7b-decode"]
    print("[workload] 7b-decode layer-wise: building", flush=True)
    model = synth.switch_model(wl)
    x, _ = synth.router_inputs(wl)
    P = len(wl.projs)
    per_layer = [[(W, A, B) for _, _, W, A, B in model[l * P:(l + 1) * P]] for l in range(wl.layers)]
    routers = [synth.normal_device((wl.d_model, wl.E), 0.02, wl.dtype, "cuda", wl.cfg_id, "Wr", l)
               for l in range(wl.layers)]
    xs = [[synth.normal_device((W.shape[1],), 1.0, wl.dtype, "cuda", wl.cfg_id, "xin", l, k)
           for k, (W, _, _) in enumerate(projs)] for l, projs in enumerate(per_layer)]
    lw = LayerwiseDecode(per_layer, routers, xs, wl.E, wl.r, wl.scale)
    assert lw.launches_per_token() == wl.layers * (2 + P * 1)
    x_tok = x[3:4].contiguous()
    lw.step(x_tok)
    torch.cuda.synchronize()
    assert lw.status() == dlm.DLM_OK
    xt = x_tok.cpu()
    agg = {"n": 0, "n_gt2ulp": 0, "max_ulp": 0}
    for l, projs in enumerate(per_layer):
        ri, rg, lg, mg, bd = oracle.pregate(xt, routers[l].cpu(), with_stats=True)
        assert (mg > 2 * bd).all(), f"layer {l}: a near tie in the router"
        assert torch.equal(lw.idx[l].cpu(), ri), f"layer {l}: router set"
        rel = (lw.g[l].cpu() - rg).abs() / rg.abs().clamp_min(1e-30)
        assert rel.max().item() <= 2.0 ** -22, f"layer {l}: router gates {rel.max()}"
        for k, ((W, A, B), xv, y) in enumerate(zip(projs, xs[l], lw.y_lora[l])):
            ref, ex, ab = oracle.sgmm(xv[None].cpu(), ri, rg, A.cpu(), B.cpu(),
                                      torch.zeros((1, W.shape[0]), dtype=wl.dtype), wl.scale, with_stats=True)
            st = check_bf16(y.cpu(), ref, ex, ab, W.shape[1] + 2 * wl.r + 2, extra=SPLIT,
                            what=f"layer-wise L{l} adapter {k}")
            agg["n"] += st["n"]
            agg["n_gt2ulp"] += st["n_gt2ulp"]
            agg["max_ulp"] = max(agg["max_ulp"], st["max_ulp"])
        if l in (0, wl.layers - 1):
            print(f"[workload] 7b-decode layer-wise: base products of layer {l}", flush=True)
            for k, ((W, _, _), xv, yb) in enumerate(zip(projs, xs[l], lw.y_base[l])):
                _, ex, ab = oracle.gemv(W.cpu(), xv.cpu(), with_stats=True)
                check_f32(yb.cpu(), ex, ab, W.shape[1], what=f"layer-wise L{l} base {k}")
    print("layer-wise adapters", agg, flush=True)
    eager = _layerwise_outputs(lw)
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(gr, stream=s):
            lw.step(x_tok, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        lw.reset_lora()
        for yl in lw.y_base:
            for y in yl:
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = _layerwise_outputs(lw)
        for a, b in zip(eager, got):
            for u, v in zip(a, b):
                for p, q in (zip(u, v) if isinstance(u, list) else [(u, v)]):
                    assert torch.equal(p, q), f"graph replay {rep} differs from the eager token"
    assert lw.status() == dlm.DLM_OK
    del gr
    # the same layers routed once per token (the first layer's router), one
    # grouped SGMM per layer: every layer's adapters use that one set
    po = LayerwiseDecode(per_layer, routers, xs, wl.E, wl.r, wl.scale, grouped=True, route_once=True)
    assert po.launches_per_token() == 1 + wl.layers * (1 + 2)
    po.step(x_tok)
    torch.cuda.synchronize()
    assert po.status() == dlm.DLM_OK
    ri, rg = oracle.pregate(xt, routers[0].cpu())
    assert torch.equal(po.idx[0].cpu(), ri)
    for l, projs in enumerate(per_layer):
        for k, ((W, A, B), xv, y) in enumerate(zip(projs, xs[l], po.y_lora[l])):
            ref, ex, ab = oracle.sgmm(xv[None].cpu(), ri, rg, A.cpu(), B.cpu(),
                                      torch.zeros((1, W.shape[0]), dtype=wl.dtype), wl.scale, with_stats=True)
            check_bf16(y.cpu(), ref, ex, ab, W.shape[1] + 2 * wl.r + 2, extra=SPLIT,
                       what=f"pre-gated unmerged L{l} adapter {k}")
        for yb, yb0 in zip(po.y_base[l], eager[3][l]):
            assert torch.equal(yb, yb0), f"layer {l}: base product differs between the two forms"
    # adapters on a second stream beside the base products: the same bits,
    # eagerly and from a graph replayed twice
    one = _layerwise_outputs(po)
    side = torch.cuda.Stream()
    po.reset_lora()
    po.step(x_tok, side=side)
    torch.cuda.synchronize()
    for u, v in zip(one[2], _layerwise_outputs(po)[2]):
        assert all(torch.equal(p, q) for p, q in zip(u, v)), "two-stream step differs"
    gr2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(gr2, stream=s):
            po.step(x_tok, stream=s, side=side)
    torch.cuda.synchronize()
    for rep in range(2):
        po.reset_lora()
        torch.cuda.synchronize()
        gr2.replay()
        torch.cuda.synchronize()
        got = _layerwise_outputs(po)
        for a, b in ((one[2], got[2]), (one[3], got[3])):
            for u, v in zip(a, b):
                assert all(torch.equal(p, q) for p, q in zip(u, v)), f"two-stream replay {rep} differs"
    del gr2
    assert po.status() == dlm.DLM_OK
    po.close()
    # the fused unmerged form: the adapters' terms inside the base product
    pf = LayerwiseDecode(per_layer, routers, xs, wl.E, wl.r, wl.scale, route_once=True, fused=True)
    assert pf.launches_per_token() == 1 + wl.layers * 2
    pf.step(x_tok)
    torch.cuda.synchronize()
    assert pf.status() == dlm.DLM_OK
    assert torch.equal(pf.idx[0].cpu(), ri)
    for l in (0, 15, wl.layers - 1):
        print(f"[workload] 7b-decode fused unmerged: layer {l}", flush=True)
        for k, ((W, A, B), xv, yb) in enumerate(zip(per_layer[l], xs[l], pf.y_base[l])):
            _, ex_w, ab_w = oracle.gemv(W.cpu(), xv.cpu(), with_stats=True)
            _, ex_a, ab_a = oracle.sgmm(xv[None].cpu(), ri, rg, A.cpu(), B.cpu(),
                                        torch.zeros((1, W.shape[0]), dtype=wl.dtype), wl.scale, with_stats=True)
            check_f32(yb.cpu(), ex_w + ex_a[0], ab_w + ab_a[0], W.shape[1] + 2 * wl.r + 32,
                      what=f"fused unmerged L{l} proj {k}")
    fused_eager = [[y.clone() for y in yl] for yl in pf.y_base]
    gr3 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(gr3, stream=s):
            pf.step(x_tok, stream=s)
    torch.cuda.synchronize()
    for rep in range(2):
        for yl in pf.y_base:
            for y in yl:
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        gr3.replay()
        torch.cuda.synchronize()
        for u, v in zip(fused_eager, pf.y_base):
            assert all(torch.equal(p, q) for p, q in zip(u, v)), f"fused replay {rep} differs"
    del gr3
    assert pf.status() == dlm.DLM_OK
    pf.close()
    lw.close()
    del model, lw, po, pf
    gc.collect()
    torch.cuda.empty_cache()


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
