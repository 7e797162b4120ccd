"""Benchmark of the pre-gated dynamic-LoRA hot path on one MI355X.

Headline (value): fused-switch weight throughput on the 7B-shaped decode
workload (32 layers x q/k/v/o 4096x4096, gate/up 4096->11008, down
11008->4096, bf16; E=8 experts of rank 16, scale 2; 256 tokens).  One step is
one pass over the token batch: the router for the 256 tokens, then the 256
fused switches (token t-1's set -> token t's set, every adapted weight of
every layer in one launch each), all with inputs resident in HBM.
value = weight bytes read + written per second (GB/s).

Beside it, in the same JSON line: SGMM tokens/s on the prefill workload (4096
tokens x 7 projections, Zipf(1.1) pairs) and on the mixed decode workload
(64 rows x 32 layers x 7 projections, 128 Markov steps); the switch kernel's
roofline (HIP-event timing of each launch on its stream, against 8 TB/s); the
same switch on the 70B-shaped workload; the router's latency at T = 1 and at
the full token counts; and the CPU oracle timed on a bounded sample of the
headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12


def _src_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


SWITCH_SOURCES = ["dynamic_lora_moe_amd/csrc/switch.hip", "dynamic_lora_moe_amd/csrc/gfx950.hpp",
                  "dynamic_lora_moe_amd/csrc/internal.hpp"]
SGMM_SOURCES = ["dynamic_lora_moe_amd/csrc/sgmm.hip", "dynamic_lora_moe_amd/csrc/sgmm.hpp",
                "dynamic_lora_moe_amd/csrc/gfx950.hpp", "dynamic_lora_moe_amd/csrc/internal.hpp"]
SGMM_PROFILE_PASSES = 3  # grouped passes per SGMM workload in --profile-kernels


def sgmm_algo_bytes(wl, idx):
    """Algorithmic bytes of one grouped SGMM pass over wl's problems for the rows'
    sets idx [T][2] (CPU): x once, y read + written, the A/B slices of the experts
    the rows use, and idx/g."""
    import numpy as np
    u = np.unique(idx.numpy())
    n_used = int((u >= 0).sum())
    per_layer = sum(wl.T * i * 2 + 2 * wl.T * o * 2 + n_used * wl.r * (i + o) * 2 for _, o, i in wl.projs)
    return per_layer * wl.layers + wl.T * 16


def _traffic(kernel_key, algo_bytes_per_launch):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    ent = t.get(kernel_key)
    if not ent or ent.get("source_hash") != _src_hash(SWITCH_SOURCES):
        return None
    return ent.get("bytes_per_launch")


def _sgmm_traffic(name):
    """HBM bytes per step of an SGMM workload (read, written, and the algorithmic
    bytes of the same profiled steps) from the committed counter summary, if it
    was taken on the current SGMM source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        ent = json.load(f).get("sgmm_" + name)
    if not ent or ent.get("source_hash") != _src_hash(SGMM_SOURCES):
        return None
    tot = ent["read_per_step"] + ent["write_per_step"]
    return {"read_per_step": ent["read_per_step"], "write_per_step": ent["write_per_step"],
            "algo_bytes_per_step": ent["algo_bytes_per_step"], "ratio": tot / ent["algo_bytes_per_step"],
            "steps_profiled": ent["passes"]}


def bench_switch(torch, dlm, synth, steps, warmup, log):
    wl = synth.WORKLOADS["7b-decode"]
    log(f"building {wl.name}: {wl.n_mats} weights, {wl.switch_w_elems() * 2 / 1e9:.2f} GB bf16")
    model = synth.switch_model(wl)
    x, Wr = synth.router_inputs(wl)
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    stream = torch.cuda.current_stream()
    T = wl.T

    def one_step(events=None):
        idx, g = dlm.pregate(x, Wr)
        L.switch(None, (idx[0], g[0]))
        for t in range(1, T):
            if events is not None:
                events[t - 1][0].record(stream)
            L.switch((idx[t - 1], g[t - 1]), (idx[t], g[t]))
            if events is not None:
                events[t - 1][1].record(stream)
        return idx

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(T - 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        one_step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for e in ev for a, b in e]
    assert L.status() == dlm.DLM_OK
    w_bytes = wl.switch_w_elems() * 2 * 2                      # read + write
    # A/B slices of the distinct experts of old and new (at most 4 experts)
    slice_bytes_per_expert = wl.layers * sum((o + i) * wl.r * 2 for _, o, i in wl.projs)
    algo_bytes = w_bytes + 4 * slice_bytes_per_expert          # router sets are top-2 distinct
    n_switch = steps * T
    ms_per_step = wall * 1e3 / steps
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    res = {
        "ms_per_step": ms_per_step,
        "weight_GBps": w_bytes * n_switch / wall / 1e9,
        "algo_GBps": algo_bytes * n_switch / wall / 1e9,
        "switch_ms": avg_launch_s * 1e3,
        "switch_ms_p50": sorted(launch_ms)[len(launch_ms) // 2],
        "switch_ms_p90": sorted(launch_ms)[int(len(launch_ms) * 0.9)],
        "algo_bytes_per_launch": algo_bytes,
        "weight_bytes_per_launch": w_bytes,
        "launches_per_switch": L.launches_per_switch(),
        "achieved_launch_GBps": algo_bytes / avg_launch_s / 1e9,
    }
    L.close()
    del model
    torch.cuda.empty_cache()
    return res


def bench_decode_loop(torch, dlm, synth, n_tokens, log):
    """Per-token decode steps on the 7B-shaped workload, on one stream:
      base:     the product of every adapted projection with the unchanged base
                weights, one launch per layer (no adapters: the reference point);
      layerwise / layerwise_grouped: per-layer routing with unmerged adapters
                (dynamic_lora_moe_amd.layerwise): per layer a router launch
                (T = 1, the layer's own router weights, the token's x), the base
                product, and the adapters as one SGMM call per projection (T = 1)
                or one grouped SGMM per layer -- W read once per token;
      pregated_unmerged: the router once per token, then per layer the base
                product and one grouped SGMM with that set;
      pregated_unmerged_2s: the same with each layer's SGMM on a second stream
                beside its base product (joined before the next layer);
      pregated_unmerged_fused: the router once per token, then per layer one
                dlm_gemv_unmerged (2 launches: the adapters' down-projections,
                then the base product with their up-projections added);
      layerwise_fused: the same with a router per layer (the layer's own
                router weights, T = 1);
      unfused:  pre-gated: router once, one switch over all 224 weights, then one
                product launch per layer (W read twice, written once: 3 x 12.95 GB);
      fused:    pre-gated: router once, then per layer the switch fused with the
                product (2 launches: W read once, written once, plus partial sums).
    Each is timed eagerly and replayed from HIP graphs (one per set-buffer parity);
    inputs are synthetic per (layer, projection), tokens come from the router's
    x.  W returns to its starting sets after each pre-gated variant (unmerge)."""
    from dynamic_lora_moe_amd.layerwise import LayerwiseDecode
    wl = synth.WORKLOADS["7b-decode"]
    log(f"decode loop: building {wl.name}")
    model = synth.switch_model(wl)
    x, Wr = synth.router_inputs(wl)
    P = len(wl.projs)
    whole = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    layers, ys = [], []
    for l in range(wl.layers):
        grp = model[l * P:(l + 1) * P]
        h = dlm.Layers([(W, A, B) for _, _, W, A, B in grp], wl.E, wl.r, wl.scale)
        xs = [synth.normal_device((W.shape[1],), 1.0, wl.dtype, "cuda", wl.cfg_id, "xin", l, k)
              for k, (_, _, W, _, _) in enumerate(grp)]
        yv = [torch.empty(W.shape[0], dtype=torch.float32, device="cuda") for _, _, W, _, _ in grp]
        h.bind_vectors(xs, yv)
        layers.append(h)
        ys.append((xs, yv))
    routers = [synth.normal_device((wl.d_model, wl.E), 0.02, wl.dtype, "cuda", wl.cfg_id, "Wr", l)
               for l in range(wl.layers)]
    per_layer = [[(W, A, B) for _, _, W, A, B in model[l * P:(l + 1) * P]] for l in range(wl.layers)]
    lw = {"layerwise": LayerwiseDecode(per_layer, routers, [xs for xs, _ in ys], wl.E, wl.r, wl.scale),
          "layerwise_grouped": LayerwiseDecode(per_layer, routers, [xs for xs, _ in ys], wl.E, wl.r, wl.scale,
                                               grouped=True),
          "pregated_unmerged": LayerwiseDecode(per_layer, routers, [xs for xs, _ in ys], wl.E, wl.r, wl.scale,
                                               grouped=True, route_once=True),
          "pregated_unmerged_fused": LayerwiseDecode(per_layer, routers, [xs for xs, _ in ys], wl.E, wl.r,
                                                     wl.scale, route_once=True, fused=True),
          "layerwise_fused": LayerwiseDecode(per_layer, routers, [xs for xs, _ in ys], wl.E, wl.r, wl.scale,
                                             fused=True)}
    x_tok = torch.empty((1, wl.d_model), dtype=wl.dtype, device="cuda")
    idx = [torch.zeros((1, 2), dtype=torch.int32, device="cuda") for _ in range(2)]
    g = [torch.zeros((1, 2), dtype=torch.float32, device="cuda") for _ in range(2)]
    s = torch.cuda.Stream()

    def step(kind, cur, first, stream):
        if kind == "base":
            for h in layers:
                h.gemv(stream=stream)
            return
        if kind in lw:
            lw[kind].step(x_tok, stream=stream)
            return
        if kind == "pregated_unmerged_2s":
            lw["pregated_unmerged"].step(x_tok, stream=stream, side=side)
            return
        dlm.pregate(x_tok, Wr, idx=idx[cur], g=g[cur], stream=stream)
        new = (idx[cur][0], g[cur][0])
        old = None if first else (idx[1 - cur][0], g[1 - cur][0])
        if kind == "unfused":
            whole.switch(old, new, stream=stream)
            for h in layers:
                h.gemv(stream=stream)
        else:
            for h in layers:
                h.switch_gemv(old, new, stream=stream)

    res = {"tokens": n_tokens}
    w_bytes = wl.switch_w_elems() * 2
    pre_gated = ("unfused", "fused")
    side = torch.cuda.Stream()
    for kind in ("base", "layerwise", "layerwise_grouped", "pregated_unmerged", "pregated_unmerged_2s",
                 "pregated_unmerged_fused", "layerwise_fused") + pre_gated:
        out = {}
        with torch.cuda.stream(s):
            # eager: token 0 from the merged-in-nothing state, then n-1 switches
            x_tok.copy_(x[0:1])
            step(kind, 0, True, s)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            for t in range(1, n_tokens):
                x_tok.copy_(x[t:t + 1])
                step(kind, t % 2, False, s)
            b.record(s)
        torch.cuda.synchronize()
        out["ms_per_token_eager"] = a.elapsed_time(b) / (n_tokens - 1)
        # graphs: one per parity of the current set buffer
        graphs = []
        for cur in (0, 1):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(gr, stream=s):
                    step(kind, cur, False, s)
            graphs.append(gr)
        torch.cuda.synchronize()
        last = (n_tokens - 1) % 2
        with torch.cuda.stream(s):
            a.record(s)
            for t in range(n_tokens):
                cur = 1 - last if t == 0 else 1 - cur
                x_tok.copy_(x[t:t + 1])
                graphs[cur].replay()
            b.record(s)
        torch.cuda.synchronize()
        out["ms_per_token_graph"] = a.elapsed_time(b) / n_tokens
        if kind == "base":
            lpt = wl.layers
        elif kind in lw:
            lpt = lw[kind].launches_per_token()
        elif kind == "pregated_unmerged_2s":
            lpt = lw["pregated_unmerged"].launches_per_token()
        else:
            lpt = 1 + (whole.launches_per_switch() + wl.layers if kind == "unfused"
                       else wl.layers * layers[0].launches_per_switch_gemv())
        out["launches_per_token"] = lpt
        out["weight_bytes_per_token"] = {"unfused": 3, "fused": 2}.get(kind, 1) * w_bytes
        out["GBps_graph"] = out["weight_bytes_per_token"] / out["ms_per_token_graph"] / 1e6
        if kind in pre_gated:
            # back to the starting weights: remove the last token's set
            cur_last = cur
            whole.switch((idx[cur_last][0], g[cur_last][0]), None)
        torch.cuda.synchronize()
        assert whole.status() == dlm.DLM_OK and all(h.status() == dlm.DLM_OK for h in layers)
        if kind in lw:
            assert lw[kind].status() == dlm.DLM_OK
        if "base" in res:
            out["time_vs_base_graph"] = out["ms_per_token_graph"] / res["base"]["ms_per_token_graph"]
        res[kind] = out
        log(f"decode loop {kind}: {out}")
        del graphs
    for h in layers:
        h.close()
    for v in lw.values():
        v.close()
    whole.close()
    del model, ys, lw
    torch.cuda.empty_cache()
    return res


def bench_switch_70b(torch, dlm, synth, n_timed, log):
    """The 70B-shaped decode workload (80 layers x q,o 8192x8192, k,v 8192->1024,
    gate,up 8192->28672, down 28672->8192; E=16, r=64): router on its 128 tokens,
    then fused switches token t-1 -> t, each launch timed with HIP events on its
    stream (2 untimed, then `n_timed`)."""
    wl = synth.WORKLOADS["70b-decode"]
    free, _ = torch.cuda.mem_get_info()
    need = wl.switch_w_elems() * 2 * 1.25
    if free < need:
        log(f"70b-decode skipped: needs {need / 2**30:.0f} GiB free, have {free / 2**30:.0f}")
        return None
    log(f"building {wl.name}: {wl.n_mats} weights, {wl.switch_w_elems() * 2 / 1e9:.2f} GB bf16")
    model = synth.switch_model(wl)
    x, Wr = synth.router_inputs(wl)
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    stream = torch.cuda.current_stream()
    idx, g = dlm.pregate(x, Wr)
    L.switch(None, (idx[0], g[0]))
    n = min(n_timed + 2, wl.T - 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for t in range(1, n + 1):
        ev[t - 1][0].record(stream)
        L.switch((idx[t - 1], g[t - 1]), (idx[t], g[t]))
        ev[t - 1][1].record(stream)
    torch.cuda.synchronize()
    assert L.status() == dlm.DLM_OK
    ms = sorted(a.elapsed_time(b) for a, b in ev[2:])
    w_bytes = wl.switch_w_elems() * 2 * 2
    slice_bytes_per_expert = wl.layers * sum((o + i) * wl.r * 2 for _, o, i in wl.projs)
    algo = w_bytes + 4 * slice_bytes_per_expert
    avg = sum(ms) / len(ms) / 1e3
    res = {"launches_timed": len(ms), "switch_ms": avg * 1e3, "switch_ms_p50": ms[len(ms) // 2],
           "switch_ms_p90": ms[int(len(ms) * 0.9)], "algo_bytes_per_launch": algo,
           "achieved_launch_GBps": algo / avg / 1e9, "frac_of_hbm_peak": algo / avg / HBM_PEAK}
    L.close()
    del model
    torch.cuda.empty_cache()
    return res


def _per_call_us(torch, call, n=20, replays=5):
    """(eager, graph) microseconds per call: n calls timed with HIP events as
    issued from Python (the binding's host work included: a short kernel then
    waits for the host), and the same n calls captured in a HIP graph and
    replayed (the device's time per call, launch gaps included)."""
    for _ in range(3):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) / n * 1e3
    s = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(gr, stream=s):
            for _ in range(n):
                call()
    torch.cuda.synchronize()
    gr.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(replays):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    graph = e0.elapsed_time(e1) / (n * replays) * 1e3
    del gr
    return eager, graph


def bench_hbm_copy(torch, log, nbytes=2 << 30, reps=10):
    """What a plain device-to-device copy (torch, bf16) achieves on this
    machine: read + write bytes per second, HIP events over `reps` copies of
    `nbytes`.  Reported beside the 8 TB/s peak, which stays the denominator."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    res = {"GBps": 2 * nbytes / sec / 1e9, "bytes_copied": nbytes, "ms_per_copy": sec * 1e3,
           "what": "torch device-to-device copy, read + write bytes per second"}
    log(f"hbm copy: {res}")
    return res


def bench_router(torch, dlm, synth, log):
    """Router latency per call at T = 1 and at the full token count of the 7B-
    and 70B-shaped workloads: from a replayed HIP graph of 20 calls (the
    device's time) and eagerly from Python (host work included)."""
    out = {}
    for name in ("7b-decode", "70b-decode"):
        wl = synth.WORKLOADS[name]
        x, Wr = synth.router_inputs(wl)
        for T in (1, wl.T):
            xt = x[:T].contiguous()
            idx = torch.empty(T, 2, dtype=torch.int32, device="cuda")
            g = torch.empty(T, 2, dtype=torch.float32, device="cuda")
            eager, us = _per_call_us(torch, lambda: dlm.pregate(xt, Wr, idx, g))
            nbytes = (xt.numel() + Wr.numel()) * xt.element_size()
            out[f"{name}_T{T}"] = {"us_per_call": us, "us_per_call_eager": eager, "GBps_x_Wr": nbytes / us / 1e3}
        # the nearest-centroid pre-gate on the same tokens: J = 4 synthetic
        # centroids per adapter, N(0, 1) like the tokens
        J = 4
        C = synth.normal_device((wl.E, J, wl.d_model), 1.0, wl.dtype, "cuda", wl.cfg_id, "centroids")
        for T in (1, wl.T):
            xt = x[:T].contiguous()
            idx = torch.empty(T, 2, dtype=torch.int32, device="cuda")
            g = torch.empty(T, 2, dtype=torch.float32, device="cuda")
            eager, us = _per_call_us(torch, lambda: dlm.pregate_centroid(xt, C, idx, g))
            out[f"{name}_centroid_J{J}_T{T}"] = {"us_per_call": us, "us_per_call_eager": eager,
                                                 "GBps_x_C": (xt.numel() + C.numel()) * xt.element_size() / us / 1e3}
    return out


def bench_sgmm(torch, dlm, synth, name, reps, log):
    wl = synth.WORKLOADS[name]
    log(f"building {name}")
    probs = synth.sgmm_problems(wl)
    idx, g = synth.batched_sets(wl)
    grp = dlm.SgmmGroup([(x, A, B, y) for _, _, x, A, B, y in probs], wl.E, wl.r, wl.scale)
    ws = grp.workspace(wl.T)
    if name == "sgmm-prefill":
        sets = [(idx.cuda(), g.cuda())]
    else:
        sets = [(idx[s].cuda(), g[s].cuda()) for s in range(wl.steps)]
    stream = torch.cuda.current_stream()

    def one():
        for i, gg in sets:
            grp.run(i, gg, workspace=ws)

    one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        one()
    e1.record(stream)
    torch.cuda.synchronize()
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    sec = e0.elapsed_time(e1) / 1e3 / reps
    tokens = wl.T * len(sets)
    nbytes = sum(sgmm_algo_bytes(wl, i.cpu()) for i, _ in sets)
    res = {"tokens_per_s": tokens / sec, "ms_per_pass": sec * 1e3, "GBps": nbytes / sec / 1e9,
           "frac_of_hbm_peak": nbytes / sec / HBM_PEAK, "algo_bytes_per_pass": nbytes,
           "traffic": _sgmm_traffic(name)}
    # spread per unit (a prefill pass, a mixed-decode step): one more round with
    # an event pair around every unit (the events add their own small gaps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sets]
    per_unit = []
    for _ in range(reps if len(sets) == 1 else 1):
        for (i, gg), (a, b) in zip(sets, evs):
            a.record(stream)
            grp.run(i, gg, workspace=ws)
            b.record(stream)
        torch.cuda.synchronize()
        per_unit += [a.elapsed_time(b) for a, b in evs]
    per_unit.sort()
    res["unit_ms_p50"] = per_unit[len(per_unit) // 2]
    res["unit_ms_p90"] = per_unit[min(len(per_unit) - 1, int(0.9 * len(per_unit)))]
    if name == "mixed-decode":
        res.update(_per_layer_variant(torch, dlm, wl, probs, sets, reps, sec, log))
        # rows that release their adapters (both slots empty) are left out by the
        # segmentation: the same steps with the upper half of the rows released
        rel = []
        for i, gg in sets:
            i2, g2 = i.clone(), gg.clone()
            i2[wl.T // 2:] = -1
            g2[wl.T // 2:] = 0
            rel.append((i2, g2))
        for i, gg in rel:
            grp.run(i, gg, workspace=ws)
        e0.record(stream)
        for _ in range(reps):
            for i, gg in rel:
                grp.run(i, gg, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        assert dlm.sgmm_status(ws) == dlm.DLM_OK
        sec_rel = e0.elapsed_time(e1) / 1e3 / reps
        res["half_released_ms_per_step"] = sec_rel * 1e3 / len(sets)
        res["half_released_time_ratio"] = sec_rel / sec
        res["grouped_ms_per_step"] = sec * 1e3 / len(sets)
    grp.close()
    del probs
    torch.cuda.empty_cache()
    return res


def _per_layer_variant(torch, dlm, wl, probs, sets, reps, sec_grouped, log):
    """The mixed decode step as one group per layer (7 projections each; 64
    rows, so each group orders its rows inside its shrink and expand: 2
    launches per layer), run eagerly and replayed from a HIP graph captured
    once (the step's sets are copied into the graph's static input buffers
    before each replay).  Beside the grouped call over all 224 projections (2
    launches per step)."""
    layers = sorted({l for l, *_ in probs})
    per = [dlm.SgmmGroup([(x, A, B, y) for l2, _, x, A, B, y in probs if l2 == l], wl.E, wl.r, wl.scale)
           for l in layers]
    wsl = [gp.workspace(wl.T) for gp in per]

    def step(i, gg, stream=None):
        for gp, w in zip(per, wsl):
            gp.run(i, gg, workspace=w, stream=stream)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps / len(sets)

    eager = timed(lambda: [step(i, gg) for i, gg in sets])
    idx_s = torch.zeros_like(sets[0][0])
    g_s = torch.zeros_like(sets[0][1])
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(idx_s, g_s, stream=side)
    torch.cuda.synchronize()

    def replay_all():
        for i, gg in sets:
            idx_s.copy_(i)
            g_s.copy_(gg)
            graph.replay()

    graphed = timed(replay_all)
    for w in wsl:
        assert dlm.sgmm_status(w) == dlm.DLM_OK
    for gp in per:
        gp.close()
    log(f"mixed decode per layer: eager {eager * 1e3:.3f} ms/step, graph {graphed * 1e3:.3f} ms/step")
    d_in_max = max(x.shape[1] for *_, x, A, B, y in probs)
    per_layer_n = len(probs) // len(layers)
    return {"launches_per_step_grouped": dlm.sgmm_launches(wl.T, d_in_max, wl.r, len(probs)),
            "launches_per_step_per_layer": len(layers) * dlm.sgmm_launches(wl.T, d_in_max, wl.r, per_layer_n),
            "per_layer_eager_ms_per_step": eager * 1e3, "per_layer_graph_ms_per_step": graphed * 1e3,
            "grouped_ms_per_step": sec_grouped * 1e3 / len(sets)}


def cpu_baseline(torch, synth, target_s, log):
    """The oracle (as it stands) on a bounded sample of the headline workload:
    the switch of every adapted weight of the first k layers, k chosen so the
    oracle runs about `target_s` seconds (at least one layer); scaled to weight
    GB/s (weight bytes read + written per second)."""
    import numpy as np

    import oracle
    wl = synth.WORKLOADS["7b-decode"]
    threads = oracle.threads()
    old = ([1, 5], [0.6, 0.4])
    new = ([2, 5], [0.7, 0.3])
    elems, secs, layers = 0, 0.0, 0
    while layers < wl.layers and (layers == 0 or secs * (layers + 1) / layers <= target_s):
        for _, _, W, A, B in synth.switch_model(wl, layers=[layers]):
            Wh, Ah, Bh = W.cpu(), A.cpu(), B.cpu()
            rows = np.arange(W.shape[0])
            t1 = time.perf_counter()
            oracle.switch_rows(Wh, rows, Ah, Bh, W.shape[0], wl.scale, old, new)
            secs += time.perf_counter() - t1
            elems += W.numel()
        layers += 1
        torch.cuda.empty_cache()
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    log(f"cpu oracle: {layers} layers, {elems} elements in {secs:.1f} s on {threads} threads ({cpu})")
    cpu = _cpu_description(cpu)
    legs = [_cpu_switch_one_thread(torch, synth, wl, old, new, log),
            _cpu_sgmm_prefill(torch, synth, log), _cpu_tiny(torch, synth, log)]
    return {"value": elems * 4 / secs / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"switch (old {old} -> new {new}) of all 7 adapted weights of the first "
                      f"{layers} of 32 layers of the 7B-shaped workload ({elems} elements, "
                      f"{secs:.1f} s of oracle time); weight bytes read+written per second, "
                      f"binary64 oracle, OpenMP over rows, {threads} threads of {cpu}",
            "cpu": cpu, "legs": legs}


def _cpu_description(model):
    """CPU model, family/model/stepping and thread count of this host."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" in ln:
                    k, v = ln.split(":", 1)
                    fields.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    fam = "/".join(fields.get(k, "?") for k in ("cpu family", "model", "stepping"))
    return f"{model} (family/model/stepping {fam}, {os.cpu_count()} logical CPUs)"


def _cpu_switch_one_thread(torch, synth, wl, old, new, log):
    """The same switch on one thread: the q and k weights of layer 0."""
    import numpy as np

    import oracle
    n0 = oracle.threads()
    oracle.set_threads(1)
    elems, secs = 0, 0.0
    try:
        for _, name, W, A, B in synth.switch_model(wl, layers=[0])[:2]:
            Wh, Ah, Bh = W.cpu(), A.cpu(), B.cpu()
            t1 = time.perf_counter()
            oracle.switch_rows(Wh, np.arange(W.shape[0]), Ah, Bh, W.shape[0], wl.scale, old, new)
            secs += time.perf_counter() - t1
            elems += W.numel()
    finally:
        oracle.set_threads(n0)
    torch.cuda.empty_cache()
    log(f"cpu oracle, one thread: {elems} elements in {secs:.1f} s")
    return {"what": "switch, one thread", "value": elems * 4 / secs / 1e9, "unit": "GB/s", "cores": 1,
            "sample": f"q and k weights of layer 0 of the 7B-shaped workload ({elems} elements, {secs:.1f} s)"}


def _cpu_sgmm_prefill(torch, synth, log):
    """The whole prefill SGMM pass (4096 tokens x 7 projections) in the oracle."""
    import oracle
    wl = synth.WORKLOADS["sgmm-prefill"]
    idx, g = synth.batched_sets(wl)
    secs = 0.0
    for _, _, x, A, B, y in synth.sgmm_problems(wl):
        xh, Ah, Bh, yh = x.cpu(), A.cpu(), B.cpu(), y.cpu()
        t1 = time.perf_counter()
        oracle.sgmm(xh, idx, g, Ah, Bh, yh, wl.scale)
        secs += time.perf_counter() - t1
    torch.cuda.empty_cache()
    log(f"cpu oracle, prefill SGMM: {secs:.2f} s")
    return {"what": "SGMM prefill pass, all threads", "value": wl.T / secs, "unit": "tokens/s",
            "cores": oracle.threads(), "seconds_per_pass": secs,
            "sample": "the whole pass: 4096 tokens x 7 projections (in full)"}


def _cpu_tiny(torch, synth, log):
    """The tiny fp32 workload in full: router on its 16 tokens and its 16 switches."""
    import oracle
    wl = synth.WORKLOADS["tiny-fp32"]
    x, Wr = synth.router_inputs(wl)
    model = [(W.cpu(), A.cpu(), B.cpu()) for _, _, W, A, B in synth.switch_model(wl)]
    t1 = time.perf_counter()
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    prev = None
    for t in range(wl.T):
        new = (ri[t].tolist(), rg[t].tolist())
        model = [(oracle.switch(W, A, B, wl.scale, prev, new), A, B) for W, A, B in model]
        prev = new
    secs = time.perf_counter() - t1
    log(f"cpu oracle, tiny fp32: {secs * 1e3:.1f} ms")
    return {"what": "tiny fp32 workload: router + 16 switches, all threads", "value": wl.T / secs,
            "unit": "switches/s", "cores": oracle.threads(), "sample": "in full"}


def profile_kernels(torch, dlm, synth, n_switch, log):
    """A short run for hardware-counter collection: the router on the 256 tokens,
    `n_switch` fused switches of the 7B-shaped workload, `n_switch` of the
    70B-shaped one (when it fits), then one 1 GiB device copy (torch) whose byte
    count calibrates the FETCH_SIZE/WRITE_SIZE counters."""
    for name in ("7b-decode", "70b-decode"):
        wl = synth.WORKLOADS[name]
        free, _ = torch.cuda.mem_get_info()
        if free < wl.switch_w_elems() * 2 * 1.25:
            log(f"{name} skipped (memory)")
            continue
        model = synth.switch_model(wl)
        x, Wr = synth.router_inputs(wl)
        L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
        idx, g = dlm.pregate(x, Wr)
        L.switch(None, (idx[0], g[0]))
        for t in range(1, n_switch):
            L.switch((idx[t - 1], g[t - 1]), (idx[t], g[t]))
        torch.cuda.synchronize()
        L.close()
        del model
        torch.cuda.empty_cache()
    # grouped SGMM: the prefill pass, then the first mixed-decode steps, each
    # SGMM_PROFILE_PASSES times (every pass starts with one segment launch)
    for name in ("sgmm-prefill", "mixed-decode"):
        wl = synth.WORKLOADS[name]
        probs = synth.sgmm_problems(wl)
        idx, g = synth.batched_sets(wl)
        grp = dlm.SgmmGroup([(x, A, B, y) for _, _, x, A, B, y in probs], wl.E, wl.r, wl.scale)
        ws = grp.workspace(wl.T)
        for p in range(SGMM_PROFILE_PASSES):
            i, gg = (idx, g) if name == "sgmm-prefill" else (idx[p], g[p])
            grp.run(i.cuda(), gg.cuda(), workspace=ws)
        torch.cuda.synchronize()
        assert dlm.sgmm_status(ws) == dlm.DLM_OK
        grp.close()
        del probs, ws
        torch.cuda.empty_cache()
    src = torch.empty(2 ** 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"profiled {n_switch} switches per workload, {SGMM_PROFILE_PASSES} passes per SGMM workload "
        f"and one copy of {src.numel() * 2} bytes")


def traffic_from(fetch_csv, write_csv, log, out_path=None):
    """Per-launch HBM bytes of the switch kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE in KiB per dispatch) of `--profile-kernels`, each
    scaled by the same counter's reading for the 1 GiB copy (known bytes);
    written to profiles/traffic.json with a hash of the kernel source."""
    import csv

    def read(path, counter, kernel):
        sw, cp = [], []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                v = float(row["Counter_Value"])
                if kernel in name:
                    sw.append(v)
                elif "copy" in name.lower() and "dlm" not in name:
                    cp.append(v)
        return sw, cp
    res = {}
    # the 7B-shaped switch (rank 16) runs switch_bf16_kernel, the 70B-shaped one
    # (rank 64) the wide-tile kernel
    for key, kernel, wl_name in (("switch_bf16_7b", "switch_bf16_kernel", "7b-decode"),
                                 ("switch_bf16_70b", "switch_wide_kernel", "70b-decode")):
        out = {}
        for part, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
            sw, cp = read(path, counter, kernel)
            if not sw:
                break
            copy_kib = max(cp)  # the 1 GiB copy is the largest copy dispatch
            factor = (2 ** 30 / 1024) / copy_kib
            out[part] = {"switch_kib_per_launch": sum(sw) / len(sw), "launches": len(sw),
                         "copy_kib": copy_kib, "scale": factor,
                         "bytes_per_launch": sum(sw) / len(sw) * 1024 * factor}
        if len(out) < 2:
            continue
        res[key] = {
            "source_hash": _src_hash(SWITCH_SOURCES), "workload": wl_name,
            "bytes_per_launch": out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"],
            "fetch": out["fetch"], "write": out["write"],
            "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                       "python3 bench.py --profile-kernels"}
    res.update(_sgmm_traffic_from(fetch_csv, write_csv, read))
    path = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    log(f"wrote {path}: {res}")


def _sgmm_traffic_from(fetch_csv, write_csv, read):
    """Per-kernel HBM bytes of the grouped SGMM passes of --profile-kernels: the
    dispatches of the SGMM kernels, in dispatch order, split into passes where a
    segmentation launch follows another kind (a pass segments with one launch,
    or with a count launch and a placing launch above 8192 rows; up to rank 64
    the shrink and expand then run as one launch) or a shrink launch follows
    anything but a segmentation (above rank 64, up to 64 rows, a pass has no
    segmentation launch: the shrink and expand order the rows); the first
    SGMM_PROFILE_PASSES passes are the prefill, the next the mixed-decode steps
    0, 1, ...  Each counter is scaled by its own reading for the 1 GiB copy."""
    import csv
    import synth
    kinds = ("segment", "shrink", "vsum", "expand", "fused")
    names = {"segment": "sgmm_seg_", "shrink": "sgmm_shrink", "vsum": "sgmm_vsum", "expand": "sgmm_expand",
             "fused": "sgmm_fused"}
    per = {}
    for part, path, counter in (("read", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        _, cp = read(path, counter, "\0")
        scale = (2 ** 30 / 1024) / max(cp) * 1024  # bytes per counted KiB
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r.get("Counter_Name") == counter
                    and any(names[k] in r.get("Kernel_Name", "") for k in kinds)]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        passes, prev = [], None
        for r in rows:
            kind = next(k for k in kinds if names[k] in r["Kernel_Name"])
            if (kind == "segment" and prev != "segment") or (kind == "shrink" and prev != "segment"):
                passes.append({})
            prev = kind
            if passes:
                passes[-1][kind] = passes[-1].get(kind, 0.0) + float(r["Counter_Value"]) * scale
        per[part] = passes
    n = SGMM_PROFILE_PASSES
    out = {}
    if len(per["read"]) < 2 * n or len(per["write"]) < 2 * n:
        return out
    for w, name in enumerate(("sgmm-prefill", "mixed-decode")):
        wl = synth.WORKLOADS[name]
        idx, _ = synth.batched_sets(wl)
        algo = [sgmm_algo_bytes(wl, idx if name == "sgmm-prefill" else idx[p]) for p in range(n)]
        ent = {"source_hash": _src_hash(SGMM_SOURCES), "workload": name, "passes": n,
               "algo_bytes_per_step": sum(algo) / n, "kernels": {}}
        for part in ("read", "write"):
            ps = per[part][w * n:(w + 1) * n]
            for k in kinds:
                v = sum(p.get(k, 0.0) for p in ps) / n
                ent["kernels"].setdefault(k, {})[part] = v
            ent[f"{part}_per_step"] = sum(sum(p.values()) for p in ps) / n
        ent["command"] = ("rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                          "python3 bench.py --profile-kernels")
        out["sgmm_" + name] = ent
    return out


def _roofline_all(sw, sw70, sg):
    """Every metric-bearing cell against 8 TB/s: the fused switch on the 7B- and
    70B-shaped workloads (per launch) and the SGMM passes (segment, shrink, K-part
    sum and expand together; per pass or step)."""
    out = [{"workload": "7b-decode", "kernel": "switch_bf16_kernel<1,256>", "bound": "hbm",
            "achieved": round(sw["achieved_launch_GBps"], 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": round(sw["achieved_launch_GBps"] * 1e9 / HBM_PEAK, 4),
            "traffic": _traffic("switch_bf16_7b", sw["algo_bytes_per_launch"]),
            "avg_launch_ms": round(sw["switch_ms"], 4)}]
    if sw70 is not None:
        out.append({"workload": "70b-decode", "kernel": "switch_wide_kernel<4,64>", "bound": "hbm",
                    "achieved": round(sw70["achieved_launch_GBps"], 1), "peak": HBM_PEAK / 1e9,
                    "unit": "GB/s", "frac": round(sw70["frac_of_hbm_peak"], 4),
                    "traffic": sw70.get("traffic"), "avg_launch_ms": round(sw70["switch_ms"], 4)})
    for key, name in (("prefill", "sgmm-prefill"), ("mixed_decode", "mixed-decode")):
        r = sg.get(key)
        if r is None:
            continue
        per = r["ms_per_pass"] if key == "prefill" else r["grouped_ms_per_step"]
        # rank 16: segment, shrink, expand; up to 64 rows no segmentation launch
        kern = ("sgmm step: segment, then shrink + expand in one launch" if key == "mixed_decode"
                else "sgmm pass: segment, then shrink + expand in one launch")
        out.append({"workload": name, "kernel": kern,
                    "bound": "hbm",
                    "achieved": round(r["GBps"], 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                    "frac": round(r["frac_of_hbm_peak"], 4),
                    "traffic": None if r.get("traffic") is None else round(
                        r["traffic"]["read_per_step"] + r["traffic"]["write_per_step"]),
                    "avg_ms": round(per, 4)})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--sgmm-reps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sgmm", action="store_true")
    ap.add_argument("--no-70b", action="store_true", help="skip the 70B-shaped switch measurement")
    ap.add_argument("--switch-70b-launches", type=int, default=32)
    ap.add_argument("--no-decode-loop", action="store_true", help="skip the per-token decode loop")
    ap.add_argument("--decode-tokens", type=int, default=64)
    ap.add_argument("--profile-kernels", type=int, nargs="?", const=4, default=0,
                    help="short run for rocprofv3 counter collection (N switches + 1 GiB copy)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter CSVs")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from, lambda m: print(f"[bench] {m}", file=sys.stderr))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the hot path here runs on a single GPU with no "
              "sharding or collectives; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_lora_moe_amd as dlm
    import synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    if args.profile_kernels:
        profile_kernels(torch, dlm, synth, args.profile_kernels, log)
        return
    copy = bench_hbm_copy(torch, log)
    sw = bench_switch(torch, dlm, synth, args.steps, args.warmup, log)
    log(f"switch: {sw}")
    dec = None
    if not args.no_decode_loop:
        dec = bench_decode_loop(torch, dlm, synth, args.decode_tokens, log)
    router = bench_router(torch, dlm, synth, log)
    log(f"router: {router}")
    sw70 = None
    if not args.no_70b:
        sw70 = bench_switch_70b(torch, dlm, synth, args.switch_70b_launches, log)
        if sw70 is not None:
            sw70["traffic"] = _traffic("switch_bf16_70b", sw70["algo_bytes_per_launch"])
        log(f"switch 70b: {sw70}")
    sg = {}
    if not args.no_sgmm:
        sg["prefill"] = bench_sgmm(torch, dlm, synth, "sgmm-prefill", args.sgmm_reps, log)
        log(f"sgmm prefill: {sg['prefill']}")
        sg["mixed_decode"] = bench_sgmm(torch, dlm, synth, "mixed-decode", max(1, args.sgmm_reps // 5), log)
        log(f"sgmm mixed decode: {sg['mixed_decode']}")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, synth, args.cpu_seconds, log)
    achieved = sw["achieved_launch_GBps"]
    out = {
        "metric": "fused-switch weight GB/s + SGMM tokens/s; fraction of MI355X HBM peak",
        "value": round(sw["weight_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sw["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "7b-decode: 32 layers x 7 adapted projections (q,k,v,o 4096x4096; "
                               "gate,up 4096->11008; down 11008->4096), E=8, r=16, scale 2, "
                               "256 tokens batch 1; step = router + 256 fused switches",
                   "tokens_per_step": 256, "weights_per_switch": 224},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(achieved * 1e9 / HBM_PEAK, 4),
                     "traffic": _traffic("switch_bf16_7b", sw["algo_bytes_per_launch"]),
                     "kernel": "switch_bf16_kernel<1,256>",
                     "avg_launch_ms": round(sw["switch_ms"], 4),
                     "algo_bytes_per_launch": sw["algo_bytes_per_launch"]},
        "roofline_all": _roofline_all(sw, sw70, sg),
        "hbm_copy_achievable": {k: (round(v, 2) if isinstance(v, float) else v) for k, v in copy.items()},
        "cpu_baseline": cpu,
        "switch": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in sw.items()},
        "switch_70b": None if sw70 is None else {k: (round(v, 4) if isinstance(v, float) else v)
                                                 for k, v in sw70.items()},
        "router": {k: {kk: round(vv, 2) for kk, vv in v.items()} for k, v in router.items()},
        "decode_loop": None if dec is None else {k: ({kk: round(vv, 4) if isinstance(vv, float) else vv
                                                      for kk, vv in v.items()} if isinstance(v, dict) else v)
                                                 for k, v in dec.items()},
        "sgmm": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                 for k, v in sg.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
