"""Fused switch parity on small and ragged shapes, invariants and the device
error path.  Every case starts from a generated pre-state (never from a state the
HIP path produced) and is compared element by element with the oracle."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth
from gpu_util import check_bf16, check_f32, dev_set, host_set

pytestmark = pytest.mark.gpu


def _model(shapes, E, r, dt, key, std=0.02):
    """[(W, A, B)] device tensors for shapes [(d_out, d_in)]."""
    out = []
    for i, (o, n) in enumerate(shapes):
        W = synth.normal_device((o, n), std, dt, "cuda", key, "W", i)
        A = synth.normal_device((E, r, n), std, dt, "cuda", key, "A", i)
        B = synth.normal_device((E, o, r), std, dt, "cuda", key, "B", i)
        out.append((W, A, B))
    return out


def _compare(model, W0s, scale, old, new, what, dt):
    """Oracle on every row of every weight from its saved pre-state."""
    stats = []
    for i, ((W, A, B), W0) in enumerate(zip(model, W0s)):
        ref, ex, ab = oracle.switch(W0, A.cpu(), B.cpu(), scale, old, new, with_stats=True)
        r = A.shape[1]
        if dt == torch.float32:
            stats.append(check_f32(W.cpu(), ex, ab, 4 * r + 2, f"{what} w{i}"))
        else:
            stats.append(check_bf16(W.cpu(), ref, ex, ab, 4 * r + 2, what=f"{what} w{i}"))
    return stats


CASES = [
    # (shapes, E, r, scale, dtype)
    ([(64, 64), (64, 64)], 4, 4, 1.0, torch.float32),                  # tiny fp32 workload shape
    ([(64, 64)], 4, 4, 2.0, torch.float32),
    ([(300, 200), (32, 64), (257, 8), (1, 64)], 8, 16, 2.0, torch.bfloat16),   # ragged rows/cols
    ([(256, 256), (512, 1024)], 8, 16, 1.0, torch.bfloat16),           # exact tiles
    ([(100, 136), (64, 72)], 4, 4, 1.0, torch.bfloat16),                # r < 16 (padded), r % 8 != 0
    ([(130, 96)], 8, 8, 1.5, torch.bfloat16),
    ([(96, 200), (520, 128)], 8, 24, 1.0, torch.bfloat16),             # r not a multiple of 16
    ([(200, 136), (64, 64)], 16, 64, 1.0, torch.bfloat16),             # 70B rank
    ([(512, 1024), (300, 1000), (256, 520)], 16, 64, 1.0, torch.bfloat16),  # wide tiles: full, ragged
    ([(520, 1536), (64, 576)], 8, 32, 2.0, torch.bfloat16),            # rank 32: odd sub-band count
    ([(257, 640), (768, 512)], 8, 48, 1.0, torch.bfloat16),            # rank 48
    # wide tiles (256 x 4096) entirely inside the weight: copy-staged from the packed A
    ([(256, 4096), (512, 8256)], 16, 64, 1.0, torch.bfloat16),         # full tiles + a ragged column band
    ([(256, 4096)], 8, 32, 2.0, torch.bfloat16),                       # rank 32 full tile
    ([(768, 4096), (300, 4096)], 8, 48, 1.0, torch.bfloat16),          # rank 48 full tiles + ragged rows
    ([(300, 1096), (16, 1032)], 4, 40, 1.0, torch.bfloat16),           # rank 40: padded ranks, d_in % 64
    ([(40, 64)], 2, 128, 0.5, torch.bfloat16),                         # largest rank
    ([(96, 200), (64, 128)], 4, 80, 1.0, torch.bfloat16),             # rank 80 (5 rank chunks)
    ([(130, 136)], 4, 96, 2.0, torch.bfloat16),                        # rank 96 (6)
    ([(70, 64), (256, 192)], 2, 100, 1.0, torch.bfloat16),            # rank 100 (7): r % 8 != 0
    ([(33, 64)], 32, 16, 1.0, torch.bfloat16),                         # most experts
    ([(40, 24), (8, 8)], 1, 1, 1.0, torch.bfloat16),                    # one expert of rank 1
    ([(5, 7)], 1, 1, 2.0, torch.float32),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_switch_parity(ci):
    shapes, E, r, scale, dt = CASES[ci]
    print(f"[switch] case {ci}: shapes={shapes} E={E} r={r} dt={dt}", flush=True)
    model = _model(shapes, E, r, dt, 1000 + ci)
    W0s = [W.cpu().clone() for W, _, _ in model]
    rng = np.random.default_rng(ci)
    L = dlm.Layers(model, E, r, scale)
    # sequence: first token from the empty set, then changes of one / both / no expert
    sets = [None]
    for _ in range(4):
        e = rng.choice(E, size=2, replace=E < 2).tolist()
        g = rng.random(2).astype(np.float32)
        g = (g / g.sum()).astype(np.float32).tolist()
        sets.append((e, g))
    sets.append((sets[-1][0][::-1], sets[-1][1][::-1]))   # same set, slots swapped
    sets.append(((sets[2][0][0], -1), (1.0, 0.0)))          # one empty slot
    for k in range(1, len(sets)):
        for (W, _, _), W0 in zip(model, W0s):
            W.copy_(W0)
        L.switch(dev_set(sets[k - 1]), dev_set(sets[k]))
        torch.cuda.synchronize()
        _compare(model, W0s, scale, sets[k - 1], sets[k], f"case{ci} step{k}", dt)
    assert L.status() == dlm.DLM_OK
    L.close()


def test_same_set_is_bitwise_noop():
    shapes = [(300, 200), (64, 4096)]
    model = _model(shapes, 8, 16, torch.bfloat16, 2001)
    W0s = [W.clone() for W, _, _ in model]
    L = dlm.Layers(model, 8, 16, 2.0)
    s = ([3, 5], [0.7, 0.3])
    L.switch(dev_set(s), dev_set(s))
    L.switch(dev_set(s), dev_set(([5, 3], [0.3, 0.7])))   # slot order does not matter
    L.switch(None, None)
    torch.cuda.synchronize()
    for (W, _, _), W0 in zip(model, W0s):
        assert torch.equal(W, W0)


def test_round_trip_and_unmerge_bound():
    shapes = [(256, 512), (96, 136)]
    E, r, scale = 8, 16, 2.0
    model = _model(shapes, E, r, torch.bfloat16, 2002)
    W0s = [W.clone() for W, _, _ in model]
    L = dlm.Layers(model, E, r, scale)
    SA, SB = ([1, 4], [0.6, 0.4]), ([7, 1], [0.55, 0.45])
    L.switch(None, dev_set(SA))
    WA = [W.clone() for W, _, _ in model]
    L.switch(dev_set(SA), dev_set(SB))
    WB = [W.clone() for W, _, _ in model]
    L.switch(dev_set(SB), dev_set(SA))
    WA2 = [W.clone() for W, _, _ in model]
    L.switch(dev_set(SA), None)
    torch.cuda.synchronize()

    def spacing(v):
        _, e = np.frexp(np.abs(v.double().cpu().numpy()))
        return np.ldexp(1.0, e - 8)

    for i, (W, A, B) in enumerate(model):
        # each switch rounds once; two roundings + fp32 accumulation bound the round trip
        _, _, ab = oracle.switch(WB[i].cpu(), A.cpu(), B.cpu(), scale, SB, SA, with_stats=True)
        bound = 0.5 * spacing(WB[i]) + 0.5 * spacing(WA2[i]) + 4 * 2.0 ** -24 * (4 * r + 2) * ab.numpy()
        diff = np.abs((WA[i].double() - WA2[i].double()).cpu().numpy())
        assert (diff <= bound).all(), f"A->B->A w{i}: max excess {(diff - bound).max()}"
        _, _, ab0 = oracle.switch(WA2[i].cpu(), A.cpu(), B.cpu(), scale, SA, None, with_stats=True)
        bound0 = 0.5 * spacing(WA2[i]) + 0.5 * spacing(W) + 4 * 2.0 ** -24 * (4 * r + 2) * ab0.numpy() \
            + np.abs((WA2[i].double() - WA[i].double()).cpu().numpy())
        diff0 = np.abs((W.double() - W0s[i].double()).cpu().numpy())
        assert (diff0 <= bound0 + 0.5 * spacing(WA[i])).all(), f"A->empty w{i}"


def test_bad_set_is_rejected_on_device_and_writes_nothing():
    model = _model([(64, 64), (96, 128)], 4, 16, torch.bfloat16, 2003)
    W0s = [W.clone() for W, _, _ in model]
    L = dlm.Layers(model, 4, 16, 1.0)
    good = dev_set(([0, 1], [0.5, 0.5]))
    for bad in [([0, 4], [0.5, 0.5]), ([-2, 1], [0.5, 0.5]), ([0, 1], [float("nan"), 0.5]),
                ([2, 3], [0.5, float("inf")])]:
        L.switch(good, dev_set(bad))
        assert L.status() == dlm.DLM_EDEVICE, bad
        for (W, _, _), W0 in zip(model, W0s):
            assert torch.equal(W, W0)
    # an unused slot may hold anything finite or not
    L.switch(dev_set(([1, -1], [0.25, float("nan")])), dev_set(([1, -1], [0.25, float("nan")])))
    assert L.status() == dlm.DLM_OK
    for (W, _, _), W0 in zip(model, W0s):
        assert torch.equal(W, W0)
    assert L.launches_per_switch() == 1


def test_switch_uses_router_output_without_host_sync():
    """End to end: the router's device output feeds the switch directly."""
    E, r, d = 8, 16, 512
    model = _model([(256, d), (384, d)], E, r, torch.bfloat16, 2004)
    W0s = [W.cpu().clone() for W, _, _ in model]
    x = synth.normal_device((2, d), 1.0, torch.bfloat16, "cuda", 2004, "x")
    Wr = synth.normal_device((d, E), 0.02, torch.bfloat16, "cuda", 2004, "Wr")
    idx, g = dlm.pregate(x, Wr)
    L = dlm.Layers(model, E, r, 2.0)
    L.switch((idx[0], g[0]), (idx[1], g[1]))
    torch.cuda.synchronize()
    # the oracle uses its own router's sets (the index decision is checked equal)
    ri, rg = oracle.pregate(x.cpu(), Wr.cpu())
    assert torch.equal(ri, idx.cpu())
    _compare(model, W0s, 2.0, host_set(ri[0], rg[0]), host_set(ri[1], rg[1]), "router->switch",
             torch.bfloat16)


def test_repack_after_changing_a_in_place():
    """Full wide tiles read the handle's packed A copy: after A changes in place,
    repack refreshes it (checked against the oracle on the new A)."""
    E, r, scale = 8, 64, 1.0
    model = _model([(256, 4096)], E, r, torch.bfloat16, 2005)
    L = dlm.Layers(model, E, r, scale)
    W, A, B = model[0]
    A.copy_(synth.normal_device(tuple(A.shape), 0.02, torch.bfloat16, "cuda", 2005, "A2", 0))
    L.repack()
    W0 = W.cpu().clone()
    s = ([2, 6], [0.6, 0.4])
    L.switch(None, dev_set(s))
    torch.cuda.synchronize()
    _compare(model, [W0], scale, None, s, "repacked A", torch.bfloat16)
    assert L.status() == dlm.DLM_OK
    L.close()
