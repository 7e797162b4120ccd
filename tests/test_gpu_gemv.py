"""Merged-weight products: dlm_gemv (y = W x) and dlm_switch_gemv (a switch, then
y = W' x with the new weights), against the oracle on generated inputs.  The
switched weights are checked as in the switch tests and must equal a plain
dlm_switch from the same pre-state bit for bit; y is checked against the
oracle's product with the oracle's own switched weights, within the fp32
summation bound plus what the switch tolerance on W' allows."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth
from gpu_util import check_bf16, check_f32, dev_set, gamma

pytestmark = pytest.mark.gpu


def _model(shapes, E, r, dt, key):
    out = []
    for i, (o, n) in enumerate(shapes):
        out.append((synth.normal_device((o, n), 0.02, dt, "cuda", key, "W", i),
                    synth.normal_device((E, r, n), 0.02, dt, "cuda", key, "A", i),
                    synth.normal_device((E, o, r), 0.02, dt, "cuda", key, "B", i)))
    return out


def _vectors(shapes, dt, key):
    xs = [synth.normal_device((n,), 1.0, dt, "cuda", key, "x", i) for i, (_, n) in enumerate(shapes)]
    ys = [torch.full((o,), float("nan"), dtype=torch.float32, device="cuda") for o, _ in shapes]
    return xs, ys


def _bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(np.maximum(e, -126) - 7), 2.0 ** -133)


def _check_y(y, W_ref, W_tol, x, what):
    """|y - W_ref x| <= gamma_n sum |W_ref x| + sum_j |x_j| (W_tol_j + the
    rounding of W_ref x itself); W_tol bounds |W' - W_ref| elementwise."""
    Wd, xd = W_ref.double().numpy(), x.detach().cpu().double().numpy()
    ref = Wd @ xd
    ab = np.abs(Wd) @ np.abs(xd)
    tol = gamma(Wd.shape[1] + 8) * ab + W_tol @ np.abs(xd) + 1e-30
    err = np.abs(y.detach().cpu().double().numpy() - ref)
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} rows out of tolerance, e.g. {np.argwhere(bad)[:5].ravel()}"


GEMV_CASES = [
    ([(300, 200), (64, 4096), (257, 8), (1, 64), (33, 11008)], torch.bfloat16),
    ([(64, 64), (37, 50)], torch.float32),
]


@pytest.mark.parametrize("ci", range(len(GEMV_CASES)))
def test_gemv_parity(ci):
    shapes, dt = GEMV_CASES[ci]
    print(f"[gemv] case {ci}: {shapes} {dt}", flush=True)
    model = _model(shapes, 4, 4, dt, 3000 + ci)
    xs, ys = _vectors(shapes, dt, 3000 + ci)
    L = dlm.Layers(model, 4, 4, 1.0)
    L.bind_vectors(xs, ys)
    L.gemv()
    torch.cuda.synchronize()
    for k, ((W, _, _), x, y) in enumerate(zip(model, xs, ys)):
        _, ex, ab = oracle.gemv(W.cpu(), x.cpu(), with_stats=True)
        check_f32(y.cpu(), ex, ab, W.shape[1] + 8, f"gemv case{ci} w{k}")
    y1 = [y.clone() for y in ys]
    L.gemv()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(y1, ys))   # bitwise reproducible
    L.close()


SWITCH_CASES = [
    # (shapes, E, r, scale, dtype): r <= 16 bf16 runs the fused kernel
    ([(300, 200), (256, 512), (64, 4096), (257, 8), (520, 776)], 8, 16, 2.0, torch.bfloat16),
    ([(100, 136), (64, 72)], 4, 4, 1.0, torch.bfloat16),
    ([(200, 136), (256, 4096)], 16, 64, 1.0, torch.bfloat16),   # wide tiles: switch, then the product
    ([(64, 64), (64, 64)], 4, 4, 1.0, torch.float32),
]


@pytest.mark.parametrize("ci", range(len(SWITCH_CASES)))
def test_switch_gemv_parity(ci):
    shapes, E, r, scale, dt = SWITCH_CASES[ci]
    print(f"[switch_gemv] case {ci}: {shapes} E={E} r={r} {dt}", flush=True)
    model = _model(shapes, E, r, dt, 3100 + ci)
    twin = [(W.clone(), A, B) for W, A, B in model]
    W0s = [W.cpu().clone() for W, _, _ in model]
    xs, ys = _vectors(shapes, dt, 3100 + ci)
    L = dlm.Layers(model, E, r, scale)
    L.bind_vectors(xs, ys)
    T = dlm.Layers(twin, E, r, scale)
    rng = np.random.default_rng(ci)
    sets = [None]
    for _ in range(3):
        e = rng.choice(E, size=2, replace=False).tolist()
        g = rng.random(2).astype(np.float32)
        sets.append((e, (g / g.sum()).astype(np.float32).tolist()))
    sets.append(((sets[-1][0][0], -1), (1.0, 0.0)))
    for k in range(1, len(sets)):
        for (W, _, _), (Wt, _, _), w0 in zip(model, twin, W0s):
            W.copy_(w0)
            Wt.copy_(w0)
        L.switch_gemv(dev_set(sets[k - 1]), dev_set(sets[k]))
        T.switch(dev_set(sets[k - 1]), dev_set(sets[k]))
        torch.cuda.synchronize()
        for i, ((W, A, B), (Wt, _, _), w0, x, y) in enumerate(zip(model, twin, W0s, xs, ys)):
            assert torch.equal(W, Wt), f"case{ci} step{k} w{i}: fused switch differs from dlm_switch"
            ref, ex, ab = oracle.switch(w0, A.cpu(), B.cpu(), scale, sets[k - 1], sets[k], with_stats=True)
            if dt == torch.bfloat16:
                check_bf16(W.cpu(), ref, ex, ab, 4 * r + 2, what=f"case{ci} step{k} w{i}")
                rd = ref.double().numpy()
                wtol = np.maximum(2 * _bf16_ulp(rd), gamma(4 * r + 2) * ab.numpy())
            else:
                check_f32(W.cpu(), ex, ab, 4 * r + 2, f"case{ci} step{k} w{i}")
                wtol = np.maximum(1e-5 * np.abs(ex.numpy()), gamma(4 * r + 2) * ab.numpy())
            _check_y(y, ref, wtol, x, f"case{ci} step{k} w{i}")
    # bitwise reproducible from the same state
    for (W, _, _), w0 in zip(model, W0s):
        W.copy_(w0)
    L.switch_gemv(None, dev_set(sets[1]))
    torch.cuda.synchronize()
    y1 = [y.clone() for y in ys]
    for (W, _, _), w0 in zip(model, W0s):
        W.copy_(w0)
    L.switch_gemv(None, dev_set(sets[1]))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(y1, ys))
    assert L.status() == dlm.DLM_OK
    L.close()
    T.close()


def test_switch_gemv_rejected_set_leaves_w_and_y():
    shapes = [(256, 512), (64, 72)]
    model = _model(shapes, 4, 16, torch.bfloat16, 3200)
    xs, ys = _vectors(shapes, torch.bfloat16, 3200)
    for y in ys:
        y.fill_(7.0)
    W0s = [W.clone() for W, _, _ in model]
    L = dlm.Layers(model, 4, 16, 1.0)
    L.bind_vectors(xs, ys)
    L.switch_gemv(None, dev_set(([1, 9], [0.5, 0.5])))   # expert 9 >= E
    torch.cuda.synchronize()
    assert L.status() == dlm.DLM_EDEVICE
    assert all(torch.equal(W, w0) for (W, _, _), w0 in zip(model, W0s))
    assert all(bool((y == 7.0).all()) for y in ys)
    L.close()


def test_gemv_requires_bound_vectors():
    model = _model([(64, 64)], 4, 4, torch.bfloat16, 3300)
    L = dlm.Layers(model, 4, 4, 1.0)
    with pytest.raises(RuntimeError):
        L.gemv()
    L.close()


def test_switch_gemv_multi_round_tail():
    """A fused launch of more tiles than the GPU keeps resident at once: 6300 x
    8264 is 25 x 33 = 825 tiles of 256 x 256, with a ragged last row band and a
    72-column edge tile.  W' must equal a plain dlm_switch bit for bit; sampled
    rows of W' and y (first band, middle, and the last two bands) are checked
    against the oracle, and y is bitwise reproducible."""
    o, n, E, r, scale = 6300, 8264, 8, 16, 2.0
    print(f"[switch_gemv] multi-round tail: {o}x{n}", flush=True)
    model = _model([(o, n)], E, r, torch.bfloat16, 3200)
    W, A, B = model[0]
    w0 = W.clone()
    twin = [(W.clone(), A, B)]
    xs, ys = _vectors([(o, n)], torch.bfloat16, 3200)
    L = dlm.Layers(model, E, r, scale)
    L.bind_vectors(xs, ys)
    T = dlm.Layers(twin, E, r, scale)
    old, new = ((1, 6), (0.625, 0.375)), ((3, 1), (0.5, 0.5))
    for k in range(2):
        W.copy_(w0)
        twin[0][0].copy_(w0)
        L.switch_gemv(dev_set(old), dev_set(new))
        T.switch(dev_set(old), dev_set(new))
        torch.cuda.synchronize()
        assert torch.equal(W, twin[0][0]), "fused switch differs from dlm_switch"
        if k == 0:
            y1 = ys[0].clone()
        else:
            assert torch.equal(y1, ys[0]), "y not bitwise reproducible"
    rows = np.array([0, 1, 255, 3000, 5887, 5888, 5900, 6143, 6144, 6200, 6299], dtype=np.int64)
    w0r = w0[torch.from_numpy(rows).cuda()].cpu()
    ref, ex, ab = oracle.switch_rows(w0r, rows, A.cpu(), B.cpu(), o, scale, old, new, with_stats=True)
    got = W[torch.from_numpy(rows).cuda()].cpu()
    check_bf16(got, ref, ex, ab, 4 * r + 2, what="multi-round tail W'")
    wtol = np.maximum(2 * _bf16_ulp(ref.double().numpy()), gamma(4 * r + 2) * ab.numpy())
    _check_y(ys[0][torch.from_numpy(rows).cuda()], ref, wtol, xs[0], "multi-round tail y")
    assert L.status() == dlm.DLM_OK
    L.close()
    T.close()
