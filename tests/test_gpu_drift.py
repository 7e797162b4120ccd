"""Drift of the in-place switch chain: W after 256 switches, each rounding once,
against the exact merge of the final set (W0 + the final set's deltas, rounded
once), for the GPU chain and for the oracle's own chain over the same switches.

Each in-place switch rounds, so the chain's result depends on its path; parity
is judged per step elsewhere.  Here the drift is reported: median / p99 / max
ulp distance of each free-run from the exact merge, the largest error in units
of ulp(0.02) (the weights' scale), and how many elements of the GPU free-run
differ from the oracle free-run by more than 2 ulp.  Only loose sanity bounds
are asserted (for bf16 storage the two chains round alike at almost every
step; for fp32 storage they part by an ulp at many steps and random-walk
apart).  Rows of W evolve independently, so the oracle follows sampled rows
exactly.  Inputs: the tiny fp32 workload (its 16 tokens cycled 16 times)
and the 7B-shaped workload (its 256 tokens; the GPU switches every weight of
all 32 layers, the oracle follows 4 rows of each projection of layers 0 and 31).
"""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth
from gpu_util import dev_set, host_set, record, sample_rows, ulp_dist_bf16

pytestmark = pytest.mark.gpu


def _f32_ordered(a: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def _ulp_f32(a, b):
    return np.abs(_f32_ordered(a) - _f32_ordered(b))


def _summary(d: np.ndarray):
    return {"median": float(np.median(d)), "p99": float(np.percentile(d, 99)), "max": int(d.max())}


def _bf(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _sets(wl, n_switch):
    x, Wr = synth.router_inputs(wl)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    T = ri.shape[0]
    return [host_set(ri[t % T], rg[t % T]) for t in range(n_switch)]


def _report(what, gpu_fr, ora_fr, exact, ulp, err_gpu, err_ora, unit):
    rep = {
        "gpu_vs_exact_ulp": _summary(ulp(gpu_fr, exact)),
        "oracle_vs_exact_ulp": _summary(ulp(ora_fr, exact)),
        "gpu_max_err_over_ulp(0.02)": float(err_gpu.max() / unit),
        "oracle_max_err_over_ulp(0.02)": float(err_ora.max() / unit),
        "gpu_vs_oracle_gt2ulp": int((ulp(gpu_fr, ora_fr) > 2).sum()),
        "n": int(exact.numel() if isinstance(exact, torch.Tensor) else exact.size),
    }
    print(f"[drift] {what}: {rep}", flush=True)
    record("drift", what, rep)
    return rep


def test_drift_tiny_fp32_256_switches():
    wl = synth.WORKLOADS["tiny-fp32"]
    sets = _sets(wl, 256)
    model = synth.switch_model(wl)
    W0 = [W.cpu().clone() for _, _, W, _, _ in model]
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    for t, s in enumerate(sets):
        L.switch(None if t == 0 else dev_set(sets[t - 1]), dev_set(s))
    torch.cuda.synchronize()
    assert L.status() == dlm.DLM_OK
    gpu, ora, ex = [], [], []
    for (_, _, W, A, B), w0 in zip(model, W0):
        Ah, Bh = A.cpu(), B.cpu()
        w = w0.clone()
        for t, s in enumerate(sets):
            w = oracle.switch(w, Ah, Bh, wl.scale, None if t == 0 else sets[t - 1], s)
        gpu.append(W.cpu().numpy())
        ora.append(w.numpy())
        ex.append(oracle.switch(w0, Ah, Bh, wl.scale, None, sets[-1]).numpy())
    L.close()
    gpu, ora, ex = (np.concatenate([a.ravel() for a in v]) for v in (gpu, ora, ex))
    unit = 2.0 ** -29  # fp32 ulp of 0.02
    rep = _report("tiny-fp32", gpu, ora, ex, _ulp_f32, np.abs(gpu - ex), np.abs(ora - ex), unit)
    # fp32 storage: each step's fp32-accumulated result may differ from the
    # correctly rounded one by an ulp, so the two chains random-walk apart; the
    # sanity bound is on the size of the drift (a few ulp per switch at most)
    assert rep["gpu_max_err_over_ulp(0.02)"] <= 4 * len(sets)
    assert rep["gpu_vs_exact_ulp"]["median"] <= 64


def test_drift_7b_decode_256_switches():
    wl = synth.WORKLOADS["7b-decode"]
    sets = _sets(wl, wl.T)
    print("[drift] 7b-decode: building", flush=True)
    model = synth.switch_model(wl)
    rng = np.random.default_rng(17)
    picked = []
    for k, (l, name, W, A, B) in enumerate(model):
        if l in (0, wl.layers - 1):
            rows = sample_rows(W.shape[0], 4, rng)
            picked.append((k, rows, W[torch.from_numpy(rows).cuda()].cpu()))
    L = dlm.Layers([(W, A, B) for _, _, W, A, B in model], wl.E, wl.r, wl.scale)
    for t, s in enumerate(sets):
        L.switch(None if t == 0 else dev_set(sets[t - 1]), dev_set(s))
    torch.cuda.synchronize()
    assert L.status() == dlm.DLM_OK
    print("[drift] 7b-decode: GPU chain done", flush=True)
    gpu, ora, ex = [], [], []
    for k, rows, w0 in picked:
        _, _, W, A, B = model[k]
        Ah, Bh = _bf(A), _bf(B)
        d_out = W.shape[0]
        w = _bf(w0)
        for t, s in enumerate(sets):
            w = _bf(oracle.switch_rows(w, rows, Ah, Bh, d_out, wl.scale, None if t == 0 else sets[t - 1], s))
        gpu.append(W[torch.from_numpy(rows).cuda()].cpu())
        ora.append(torch.from_numpy(w.view(np.int16)).view(torch.bfloat16))
        ex.append(oracle.switch_rows(_bf(w0), rows, Ah, Bh, d_out, wl.scale, None, sets[-1]))
    L.close()
    del model
    torch.cuda.empty_cache()
    gpu, ora, ex = (torch.cat([a.reshape(-1) for a in v]) for v in (gpu, ora, ex))
    unit = 2.0 ** -13  # bf16 ulp of 0.02
    e = ex.double().numpy()
    rep = _report("7b-decode (layers 0 and 31, 4 rows per projection)", gpu, ora, ex, ulp_dist_bf16,
                  np.abs(gpu.double().numpy() - e), np.abs(ora.double().numpy() - e), unit)
    assert rep["gpu_vs_oracle_gt2ulp"] <= 0.01 * rep["n"]
    assert rep["gpu_vs_exact_ulp"]["median"] <= 16
