"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph over the library's
launches on the capturing stream): every replay must give the same bits as the
same calls made eagerly.  Replays run several times in a row, with eager work,
synchronisations and new input sets between them (the sets live in static
device buffers the graph reads)."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import synth

pytestmark = pytest.mark.gpu


def _sets(T, E, rng):
    idx = np.full((T, 2), -1, np.int32)
    g = np.zeros((T, 2), np.float32)
    for t in range(T):
        k = rng.integers(1, 3)
        e = rng.choice(E, size=k, replace=False)
        idx[t, :k] = e
        w = rng.random(k).astype(np.float32)
        g[t, :k] = w / w.sum()
    return torch.from_numpy(idx), torch.from_numpy(g)


@pytest.mark.parametrize("r", [16, 64, 128])
def test_switch_graph_replays_match_eager(r):
    """Rank 16: the 256-wide tiles; 64: the wide tiles (packed A images); 128:
    64-wide tiles whose LDS needs the raised limit (set when the handle is made,
    so the captured launch is a launch only)."""
    shapes = [(256, 512), (300, 264), (1024, 1024)]
    E, scale = 8, 2.0
    model = []
    for i, (o, n) in enumerate(shapes):
        model.append((synth.normal_device((o, n), 0.02, torch.bfloat16, "cuda", 5000, "W", i),
                      synth.normal_device((E, r, n), 0.02, torch.bfloat16, "cuda", 5000, "A", i),
                      synth.normal_device((E, o, r), 0.02, torch.bfloat16, "cuda", 5000, "B", i)))
    W0 = [W.clone() for W, _, _ in model]
    L = dlm.Layers(model, E, r, scale)
    old_i = torch.zeros(2, dtype=torch.int32, device="cuda")
    old_g = torch.zeros(2, dtype=torch.float32, device="cuda")
    new_i = torch.zeros(2, dtype=torch.int32, device="cuda")
    new_g = torch.zeros(2, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(3)

    def draw():
        e = rng.choice(E, size=4, replace=False)
        w = rng.random(4).astype(np.float32)
        return ((e[:2].tolist(), (w[:2] / w[:2].sum()).tolist()), (e[2:].tolist(), (w[2:] / w[2:].sum()).tolist()))

    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            L.switch((old_i, old_g), (new_i, new_g), stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        old, new = draw()
        for (W, _, _), w0 in zip(model, W0):
            W.copy_(w0)
        old_i.copy_(torch.tensor(old[0], dtype=torch.int32))
        old_g.copy_(torch.tensor(old[1], dtype=torch.float32))
        new_i.copy_(torch.tensor(new[0], dtype=torch.int32))
        new_g.copy_(torch.tensor(new[1], dtype=torch.float32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [W.clone() for W, _, _ in model]
        for (W, _, _), w0 in zip(model, W0):
            W.copy_(w0)
        L.switch((old_i, old_g), (new_i, new_g))
        torch.cuda.synchronize()
        for k, ((W, _, _), gw) in enumerate(zip(model, got)):
            assert torch.equal(W, gw), (rep, k)
    assert L.status() == dlm.DLM_OK
    L.close()


def test_sgmm_per_layer_groups_in_graph_match_grouped_eager():
    """Per-layer groups (one segmentation per layer) captured in one graph give
    the same bits as one group over all layers run eagerly: the rows and their
    sets, hence tiles and unions, are the same for every layer."""
    T, E, r, layers = 64, 8, 16, 4
    shapes = [(256, 256), (512, 256), (256, 512)]
    probs = []
    for l in range(layers):
        for p, (n, o) in enumerate(shapes):
            key = (6000, l, p)
            probs.append((synth.normal_device((T, n), 1.0, torch.bfloat16, "cuda", *key, "x"),
                          synth.normal_device((E, r, n), 0.02, torch.bfloat16, "cuda", *key, "A"),
                          synth.normal_device((E, o, r), 0.02, torch.bfloat16, "cuda", *key, "B"),
                          synth.normal_device((T, o), 0.3, torch.bfloat16, "cuda", *key, "y")))
    y0 = [p[3].clone() for p in probs]
    per_layer = [dlm.SgmmGroup(probs[l * len(shapes):(l + 1) * len(shapes)], E, r, 1.0)
                 for l in range(layers)]
    ws = [grp.workspace(T) for grp in per_layer]
    whole = dlm.SgmmGroup(probs, E, r, 1.0)
    ws_whole = whole.workspace(T)
    idx_s = torch.zeros(T, 2, dtype=torch.int32, device="cuda")
    g_s = torch.zeros(T, 2, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for grp, w in zip(per_layer, ws):
                grp.run(idx_s, g_s, T, workspace=w, stream=s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    for rep in range(4):
        idx, g = _sets(T, E, rng)
        idx_s.copy_(idx)
        g_s.copy_(g)
        for (_, _, _, y), y00 in zip(probs, y0):
            y.copy_(y00)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [p[3].clone() for p in probs]
        for (_, _, _, y), y00 in zip(probs, y0):
            y.copy_(y00)
        whole.run(idx_s, g_s, T, workspace=ws_whole)
        torch.cuda.synchronize()
        for k, (p, gy) in enumerate(zip(probs, got)):
            assert torch.equal(p[3], gy), (rep, k)
        assert all(dlm.sgmm_status(w) == dlm.DLM_OK for w in ws)
    for grp in per_layer:
        grp.close()
    whole.close()


def test_switch_gemv_per_layer_graph_replays_match_eager():
    """Two 'layers', each switched and multiplied by its bound inputs with
    dlm_switch_gemv, captured in one graph: every replay gives the weights and
    products of the same calls made eagerly."""
    E, r = 8, 16
    shapes = [(256, 512), (300, 264)]
    layers, W0, vecs = [], [], []
    for l in range(2):
        m = [(synth.normal_device((o, n), 0.02, torch.bfloat16, "cuda", 7000, "W", l, i),
              synth.normal_device((E, r, n), 0.02, torch.bfloat16, "cuda", 7000, "A", l, i),
              synth.normal_device((E, o, r), 0.02, torch.bfloat16, "cuda", 7000, "B", l, i))
             for i, (o, n) in enumerate(shapes)]
        xs = [synth.normal_device((n,), 1.0, torch.bfloat16, "cuda", 7000, "x", l, i) for i, (_, n) in enumerate(shapes)]
        ys = [torch.zeros(o, dtype=torch.float32, device="cuda") for o, _ in shapes]
        h = dlm.Layers(m, E, r, 2.0)
        h.bind_vectors(xs, ys)
        layers.append((h, m, ys))
        W0.append([W.clone() for W, _, _ in m])
    old_i = torch.zeros(2, dtype=torch.int32, device="cuda")
    old_g = torch.zeros(2, dtype=torch.float32, device="cuda")
    new_i = torch.zeros(2, dtype=torch.int32, device="cuda")
    new_g = torch.zeros(2, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for h, _, _ in layers:
                h.switch_gemv((old_i, old_g), (new_i, new_g), stream=s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)

    def reset():
        for (_, m, ys), w0 in zip(layers, W0):
            for (W, _, _), w in zip(m, w0):
                W.copy_(w)
            for y in ys:
                y.zero_()

    for rep in range(4):
        e = rng.choice(E, size=4, replace=False)
        w = rng.random(4).astype(np.float32)
        old_i.copy_(torch.tensor(e[:2].tolist(), dtype=torch.int32))
        old_g.copy_(torch.tensor((w[:2] / w[:2].sum()).tolist(), dtype=torch.float32))
        new_i.copy_(torch.tensor(e[2:].tolist(), dtype=torch.int32))
        new_g.copy_(torch.tensor((w[2:] / w[2:].sum()).tolist(), dtype=torch.float32))
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [([W.clone() for W, _, _ in m], [y.clone() for y in ys]) for _, m, ys in layers]
        reset()
        for h, _, _ in layers:
            h.switch_gemv((old_i, old_g), (new_i, new_g))
        torch.cuda.synchronize()
        for (h, m, ys), (gw, gy) in zip(layers, got):
            assert all(torch.equal(W, a) for (W, _, _), a in zip(m, gw)), rep
            assert all(torch.equal(y, a) for y, a in zip(ys, gy)), rep
    for h, _, _ in layers:
        assert h.status() == dlm.DLM_OK
        h.close()


# ---- launch counts: the kernel nodes of a captured call -----------------------

_HIP = None


def _kernel_nodes(graph) -> int:
    """Kernel nodes of a captured (not instantiated) graph, read with
    hipGraphGetNodes / hipGraphNodeGetType (hipGraphNodeTypeKernel = 0)."""
    import ctypes
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
    h = ctypes.c_void_p(graph.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert _HIP.hipGraphGetNodes(h, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * max(n.value, 1))()
    assert _HIP.hipGraphGetNodes(h, nodes, ctypes.byref(n)) == 0
    kernels = 0
    for i in range(n.value):
        kind = ctypes.c_int(-1)
        assert _HIP.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(kind)) == 0
        kernels += kind.value == 0
    return kernels


def _captured(fn) -> int:
    """Kernel launches fn makes, counted from a capture of it (never replayed)."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(g):
        fn()
    n = _kernel_nodes(g)
    g.reset()
    return n


@pytest.mark.parametrize("T,shapes,E,r,dt,group,want", [
    (2, [(4104, 1032)], 8, 16, torch.bfloat16, False, 1),                       # few rows, one launch
    (3, [(4104, 1032), (200, 264), (11008, 4096)], 8, 16, torch.bfloat16, True, 2),  # few rows, a group
    (64, [(4104, 200), (2056, 64)], 8, 16, torch.bfloat16, True, 2),           # rows ordered in the kernels
    (65, [(4104, 200), (2056, 64)], 8, 16, torch.bfloat16, True, 3),           # segment, shrink, expand
    (8192, [(4104, 200)], 8, 16, torch.bfloat16, False, 2),                    # 256 pairs: segment, shrink + expand
    (64, [(4104, 72)], 4, 80, torch.bfloat16, False, 4),                        # + the K-slice sum (r > 64)
    (9000, [(64, 72)], 8, 16, torch.bfloat16, False, 3),                        # + the count launch (T > 8192)
    (40, [(72, 40)], 4, 8, torch.float32, False, 3),                            # fp32
])
def test_sgmm_launch_count_matches_captured_kernels(T, shapes, E, r, dt, group, want):
    """dlm_sgmm_launches (the count the layer-wise decode and the bench report)
    equals the kernel nodes a capture of the call records."""
    from test_gpu_sgmm import _problem, _sets as _sgmm_sets
    print(f"[graph] launch count T={T} shapes={shapes} r={r} {dt} group={group}", flush=True)
    probs = [_problem(T, i, o, E, r, dt, 5100 + k) for k, (i, o) in enumerate(shapes)]
    idx, g = _sgmm_sets(T, E, np.random.default_rng(5200))
    idx, g = idx.cuda(), g.cuda()
    d_in_max = max(i for i, _ in shapes)
    assert dlm.sgmm_launches(T, d_in_max, r, len(shapes), dt) == want
    if group:
        grp = dlm.SgmmGroup(probs, E, r, 1.0)
        ws = grp.workspace(T)
        grp.run(idx, g, workspace=ws)  # first call outside the capture
        assert _captured(lambda: grp.run(idx, g, workspace=ws)) == want
        grp.close()
    else:
        (x, A, B, y), = probs
        ws = dlm.sgmm_workspace(T, shapes[0][0], E, r)
        dlm.sgmm(x, idx, g, A, B, y, 1.0, ws)
        assert _captured(lambda: dlm.sgmm(x, idx, g, A, B, y, 1.0, ws)) == want
    assert dlm.sgmm_status(ws) == dlm.DLM_OK


def test_switch_launch_counts_match_captured_kernels():
    """dlm_switch: one launch for every weight of every layer; dlm_switch_gemv
    and dlm_gemv_unmerged: the counted two; dlm_gemv: one."""
    print("[graph] switch launch counts", flush=True)
    E, r = 4, 16
    shapes = [(264, 512), (512, 264), (96, 1040)]
    model = []
    for k, (o, i) in enumerate(shapes):
        W = synth.normal_device((o, i), 0.05, torch.bfloat16, "cuda", (5300, k), "W")
        A = synth.normal_device((E, r, i), 0.05, torch.bfloat16, "cuda", (5300, k), "A")
        B = synth.normal_device((E, o, r), 0.05, torch.bfloat16, "cuda", (5300, k), "B")
        model.append((W, A, B))
    L = dlm.Layers(model, E, r, 1.0)
    xs = [synth.normal_device((i,), 1.0, torch.bfloat16, "cuda", (5301, k), "x") for k, (_, i) in enumerate(shapes)]
    ys = [torch.zeros(o, dtype=torch.float32, device="cuda") for o, _ in shapes]
    L.bind_vectors(xs, ys)
    new = (torch.tensor([1, 3], dtype=torch.int32, device="cuda"), torch.tensor([0.6, 0.4], device="cuda"))
    old = (torch.tensor([0, -1], dtype=torch.int32, device="cuda"), torch.tensor([1.0, 0.0], device="cuda"))
    L.switch(None, old)
    assert _captured(lambda: L.switch(old, new)) == L.launches_per_switch() == 1
    assert _captured(lambda: L.switch_gemv(old, new)) == L.launches_per_switch_gemv() == 2
    assert _captured(lambda: L.gemv()) == 1
    assert _captured(lambda: L.gemv_unmerged(new)) == L.launches_per_gemv_unmerged() == 2
    assert L.status() == dlm.DLM_OK
    L.close()


@pytest.mark.parametrize("T,n_prob", [(64, 128), (300, 26)])
def test_sgmm_one_launch_group_in_graph_matches_eager(T, n_prob):
    """A group of at least 256 (problem, tile) pairs runs its shrink and expand
    in one launch, each XCD's expand items waiting on that XCD's shrink items.
    Captured in a HIP graph and replayed (where the device starts the launch's
    workgroups on another XCD than eagerly), every replay, with eager work in
    between, must give the eager launch's bits and leave the status word clear
    (it is set if an expand item's shrink items ran on another XCD)."""
    E, r = 8, 16
    assert n_prob * ((T + 31) // 32) >= 256
    print(f"[graph] one-launch SGMM group T={T} problems={n_prob}", flush=True)
    shapes = [(136, 64), (64, 1032), (2056, 72)]
    probs = []
    for p in range(n_prob):
        n, o = shapes[p % len(shapes)]
        key = (6100, T, p)
        probs.append((synth.normal_device((T, n), 1.0, torch.bfloat16, "cuda", *key, "x"),
                      synth.normal_device((E, r, n), 0.02, torch.bfloat16, "cuda", *key, "A"),
                      synth.normal_device((E, o, r), 0.02, torch.bfloat16, "cuda", *key, "B"),
                      synth.normal_device((T, o), 0.3, torch.bfloat16, "cuda", *key, "y")))
    assert dlm.sgmm_launches(T, 2056, r, n_prob) == 2
    y0 = [p[3].clone() for p in probs]
    grp = dlm.SgmmGroup(probs, E, r, 1.0)
    ws = grp.workspace(T)
    idx_s = torch.zeros(T, 2, dtype=torch.int32, device="cuda")
    g_s = torch.zeros(T, 2, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            grp.run(idx_s, g_s, T, workspace=ws, stream=s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for rep in range(3):
        idx, g = _sets(T, E, rng)
        idx_s.copy_(idx)
        g_s.copy_(g)
        for (_, _, _, y), y00 in zip(probs, y0):
            y.copy_(y00)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert dlm.sgmm_status(ws) == dlm.DLM_OK, rep
        got = [p[3].clone() for p in probs]
        for (_, _, _, y), y00 in zip(probs, y0):
            y.copy_(y00)
        grp.run(idx_s, g_s, T, workspace=ws)
        torch.cuda.synchronize()
        assert dlm.sgmm_status(ws) == dlm.DLM_OK, rep
        for k, (p, gy) in enumerate(zip(probs, got)):
            assert torch.equal(p[3], gy), (rep, k)
    grp.close()
