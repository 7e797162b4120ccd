"""The decode product with one set's adapters unmerged (dlm_gemv_unmerged):
y = W x + s sum_k g_k B_k (A_k x) for every weight of a handle, against the
oracle's product and its unmerged adapters at T = 1, added in binary64.

Tolerance: fp32 y against the exact sum, |y - exact| <= gamma_n S with S the
sum of the magnitudes of every term (the product's sum |W_j x_j| plus the
SGMM oracle's sum |s g_k| sum_rho |B_rho| sum_j |x_j A_rho,j|) and
n = d_in + 2r + 32: the row's chains and butterfly (d_in + 8), the rank
vectors' chains, butterfly, waves and slices (d_in + 16), two products per term,
the terms' chain and butterfly, and the final add."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth
from gpu_util import check_f32

pytestmark = pytest.mark.gpu


def _model(shapes, E, r, dt, key):
    return [(synth.normal_device((o, n), 0.02, dt, "cuda", key, "W", i),
             synth.normal_device((E, r, n), 0.02, dt, "cuda", key, "A", i),
             synth.normal_device((E, o, r), 0.02, dt, "cuda", key, "B", i)) for i, (o, n) in enumerate(shapes)]


def _vectors(shapes, dt, key):
    xs = [synth.normal_device((n,), 1.0, dt, "cuda", key, "x", i) for i, (_, n) in enumerate(shapes)]
    ys = [torch.full((o,), float("nan"), dtype=torch.float32, device="cuda") for o, _ in shapes]
    return xs, ys


def _check(model, xs, ys, s, E, r, scale, what):
    idx = torch.tensor([s[0]], dtype=torch.int32)
    g = torch.tensor([s[1]], dtype=torch.float32)
    for k, ((W, A, B), x, y) in enumerate(zip(model, xs, ys)):
        _, ex_w, ab_w = oracle.gemv(W.cpu(), x.cpu(), with_stats=True)
        y0 = torch.zeros((1, W.shape[0]), dtype=W.dtype)
        _, ex_a, ab_a = oracle.sgmm(x.cpu()[None], idx, g, A.cpu(), B.cpu(), y0, scale, with_stats=True)
        check_f32(y.cpu(), ex_w + ex_a[0], ab_w + ab_a[0], W.shape[1] + 2 * r + 32, f"{what} w{k}")


UNMERGED_CASES = [
    # (shapes [(d_out, d_in)], E, r, scale, dtype, set)
    ([(300, 200), (256, 512), (64, 4096), (257, 8), (520, 776), (33, 11008)], 8, 16, 2.0, torch.bfloat16,
     ([3, 5], [0.7, 0.3])),
    ([(96, 8192), (40, 2056)], 16, 64, 1.0, torch.bfloat16, ([7, 0], [0.55, 0.45])),   # two terms per lane
    ([(50, 4104)], 4, 128, 0.5, torch.bfloat16, ([1, 2], [0.6, 0.4])),                  # four terms per lane
    ([(64, 4096), (24, 16)], 8, 24, 1.0, torch.bfloat16, ([6, -1], [1.0, 0.0])),         # one empty slot, r % 16
    ([(72, 2064)], 8, 16, 1.5, torch.bfloat16, ([4, 4], [0.5, 0.5])),                    # a duplicated expert
    ([(64, 64), (37, 50)], 4, 4, 1.0, torch.float32, ([2, 0], [0.8, 0.2])),             # fp32
    ([(200, 20000)], 4, 8, 1.0, torch.bfloat16, ([0, 3], [0.3, 0.7])),                  # 10 K slices (past 8 ahead)
]


@pytest.mark.parametrize("ci", range(len(UNMERGED_CASES)))
def test_gemv_unmerged_parity(ci):
    shapes, E, r, scale, dt, s = UNMERGED_CASES[ci]
    print(f"[unmerged] case {ci}: {shapes} E={E} r={r} {dt} set={s}", flush=True)
    model = _model(shapes, E, r, dt, 4100 + ci)
    W0 = [W.clone() for W, _, _ in model]
    xs, ys = _vectors(shapes, dt, 4100 + ci)
    L = dlm.Layers(model, E, r, scale)
    L.bind_vectors(xs, ys)
    st = (torch.tensor(s[0], dtype=torch.int32, device="cuda"), torch.tensor(s[1], dtype=torch.float32, device="cuda"))
    L.gemv_unmerged(st)
    assert L.status() == dlm.DLM_OK
    _check(model, xs, ys, s, E, r, scale, f"unmerged case{ci}")
    assert all(torch.equal(W, w0) for (W, _, _), w0 in zip(model, W0))   # W untouched
    y1 = [y.clone() for y in ys]
    # bitwise reproducible, and the same with the set's slots swapped
    sw = (st[0].flip(0).contiguous(), st[1].flip(0).contiguous())
    L.gemv_unmerged(sw)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(y1, ys))
    assert L.launches_per_gemv_unmerged() == 2
    L.close()


def test_gemv_unmerged_empty_set_is_the_product():
    """The empty set (both slots -1) gives exactly dlm_gemv's y."""
    shapes = [(300, 200), (64, 4096), (33, 11008)]
    model = _model(shapes, 8, 16, torch.bfloat16, 4200)
    xs, ys = _vectors(shapes, torch.bfloat16, 4200)
    L = dlm.Layers(model, 8, 16, 2.0)
    L.bind_vectors(xs, ys)
    L.gemv()
    torch.cuda.synchronize()
    y_base = [y.clone() for y in ys]
    st = (torch.tensor([-1, -1], dtype=torch.int32, device="cuda"), torch.zeros(2, device="cuda"))
    L.gemv_unmerged(st)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(y_base, ys))
    L.close()


def test_gemv_unmerged_bad_set_leaves_y_and_sets_status():
    shapes = [(64, 4096), (33, 520)]
    model = _model(shapes, 8, 16, torch.bfloat16, 4300)
    xs, ys = _vectors(shapes, torch.bfloat16, 4300)
    L = dlm.Layers(model, 8, 16, 1.0)
    L.bind_vectors(xs, ys)
    good = ([2, 1], [0.6, 0.4])
    dgood = (torch.tensor(good[0], dtype=torch.int32, device="cuda"), torch.tensor(good[1], device="cuda"))
    L.gemv_unmerged(dgood)
    assert L.status() == dlm.DLM_OK
    before = [y.clone() for y in ys]
    for bad_i, bad_g in (([8, 1], [0.5, 0.5]), ([2, -3], [0.5, 0.5]), ([2, 1], [float("nan"), 0.5])):
        st = (torch.tensor(bad_i, dtype=torch.int32, device="cuda"), torch.tensor(bad_g, dtype=torch.float32, device="cuda"))
        L.gemv_unmerged(st)
        assert L.status() == dlm.DLM_EDEVICE
        assert all(torch.equal(a, b) for a, b in zip(before, ys))
    # the status word was cleared: a good set works again on the same handle
    L.gemv_unmerged(dgood)
    assert L.status() == dlm.DLM_OK
    _check(model, xs, ys, good, 8, 16, 1.0, "after bad sets")
    L.close()


def test_gemv_unmerged_more_than_64_weights():
    """A handle of 70 weights: past 64 descriptors the first launch finds each
    K slice's weight by a ballot per 64 keys instead of one lane per
    descriptor.  Weights 62-66 span several K slices, so slices on both sides
    of the 64-descriptor boundary belong to multi-slice weights."""
    rng = np.random.default_rng(4400)
    shapes = []
    for i in range(70):
        d_in = 8 * int(rng.integers(260, 700)) if 62 <= i <= 66 else 8 * int(rng.integers(1, 64))
        shapes.append((int(rng.integers(1, 48)), d_in))
    model = _model(shapes, 8, 16, torch.bfloat16, 4400)
    xs, ys = _vectors(shapes, torch.bfloat16, 4400)
    L = dlm.Layers(model, 8, 16, 1.5)
    L.bind_vectors(xs, ys)
    s = ([5, 2], [0.35, 0.65])
    L.gemv_unmerged((torch.tensor(s[0], dtype=torch.int32, device="cuda"),
                     torch.tensor(s[1], dtype=torch.float32, device="cuda")))
    assert L.status() == dlm.DLM_OK
    _check(model, xs, ys, s, 8, 16, 1.5, "70 weights")
    L.close()


def test_gemv_unmerged_requires_bound_vectors_and_follows_a_rebind():
    """Without bound vectors the call is refused before anything is enqueued;
    after a second binding (new vectors, the partials buffer reallocated) the
    product uses the new vectors."""
    shapes = [(64, 4104), (40, 16)]
    model = _model(shapes, 8, 16, torch.bfloat16, 4500)
    L = dlm.Layers(model, 8, 16, 1.0)
    s = ([1, 6], [0.25, 0.75])
    st = (torch.tensor(s[0], dtype=torch.int32, device="cuda"), torch.tensor(s[1], dtype=torch.float32, device="cuda"))
    with pytest.raises(RuntimeError):
        L.gemv_unmerged(st)
    xs, ys = _vectors(shapes, torch.bfloat16, 4500)
    L.bind_vectors(xs, ys)
    L.gemv_unmerged(st)
    assert L.status() == dlm.DLM_OK
    _check(model, xs, ys, s, 8, 16, 1.0, "first binding")
    xs2, ys2 = _vectors(shapes, torch.bfloat16, 4501)
    L.bind_vectors(xs2, ys2)
    before = [y.clone() for y in ys]
    L.gemv_unmerged(st)
    assert L.status() == dlm.DLM_OK
    _check(model, xs2, ys2, s, 8, 16, 1.0, "second binding")
    assert all(torch.equal(a, b) for a, b in zip(before, ys))  # the old outputs are left alone
    L.close()
