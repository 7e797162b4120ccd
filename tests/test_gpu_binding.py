"""The binding refuses buffers whose shape, dtype or device do not match what the
library will assume (the C ABI takes bare pointers and cannot check extents).
Every case raises in Python before any call into the library."""
import pytest
import torch

import dynamic_lora_moe_amd as dlm

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_sgmm_rejects_mismatched_buffers():
    T, d_in, d_out, E, r = 8, 64, 32, 4, 16
    x, A, B, y = _t(T, d_in), _t(E, r, d_in), _t(E, d_out, r), _t(T, d_out)
    idx = torch.tensor([[0, 1]] * T, dtype=torch.int32, device="cuda")
    g = torch.zeros((T, 2), dtype=torch.float32, device="cuda")
    dlm.sgmm(x, idx, g, A, B, y, 1.0)          # the matching call goes through
    torch.cuda.synchronize()
    bad = [
        dict(B=_t(E, d_out, r + 1)),           # B's rank does not match A's
        dict(B=_t(E - 1, d_out, r)),           # fewer experts in B than in A
        dict(y=_t(T - 1, d_out)),              # y holds fewer rows than x
        dict(y=_t(T, d_out, dtype=torch.float32)),
        dict(idx=idx[: T - 1]),                # a set per row is needed
        dict(idx=idx.to(torch.int64)),
        dict(g=g.t().contiguous()),
        dict(A=_t(E, r, d_in + 8)),
    ]
    for kw in bad:
        args = dict(x=x, idx=idx, g=g, A=A, B=B, y=y)
        args.update(kw)
        with pytest.raises(ValueError):
            dlm.sgmm(args["x"], args["idx"], args["g"], args["A"], args["B"], args["y"], 1.0)


def test_group_rejects_more_rows_than_its_problems_hold():
    E, r = 4, 16
    probs = [(_t(16, 64), _t(E, r, 64), _t(E, 32, r), _t(16, 32)),
             (_t(12, 64), _t(E, r, 64), _t(E, 48, r), _t(12, 48))]
    grp = dlm.SgmmGroup(probs, E, r, 1.0)
    try:
        idx = torch.full((16, 2), -1, dtype=torch.int32, device="cuda")
        g = torch.zeros((16, 2), dtype=torch.float32, device="cuda")
        with pytest.raises(ValueError):
            grp.run(idx, g)                    # 16 rows, the second problem holds 12
        ws = grp.run(idx[:12], g[:12])         # 12 rows is fine
        assert dlm.sgmm_status(ws) == dlm.DLM_OK
        with pytest.raises(ValueError):
            grp.run(idx, g[:8], T=12)          # g shorter than T
    finally:
        grp.close()
    with pytest.raises(ValueError):
        dlm.SgmmGroup([(_t(16, 64), _t(E, r, 64), _t(E, 32, r), _t(15, 32))], E, r, 1.0)


def test_layers_reject_mismatched_adapters():
    E, r = 4, 16
    W = _t(64, 128)
    with pytest.raises(ValueError):
        dlm.Layers([(W, _t(E, r, 64), _t(E, 64, r))], E, r, 1.0)      # A's d_in is not W's
    with pytest.raises(ValueError):
        dlm.Layers([(W, _t(E, r, 128), _t(E, 64, r))], E, r + 16, 1.0)  # handle rank differs
    L = dlm.Layers([(W, _t(E, r, 128), _t(E, 64, r))], E, r, 1.0)
    try:
        with pytest.raises(ValueError):
            L.bind_vectors([_t(64)], [_t(64, dtype=torch.float32)])       # x must be [d_in]
        with pytest.raises(ValueError):
            L.bind_vectors([_t(128)], [_t(64)])                            # y must be fp32
    finally:
        L.close()


def test_pregate_rejects_short_outputs():
    x, Wr = _t(8, 64), _t(64, 4)
    idx, g = dlm.pregate(x, Wr)
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        dlm.pregate(x, Wr, idx=idx[:4])
    with pytest.raises(ValueError):
        dlm.pregate(x, Wr, g=g.to(torch.bfloat16))
    with pytest.raises(ValueError):
        dlm.pregate(x, _t(32, 4))


def test_aliased_buffers_are_refused_before_launch():
    """A set stored inside a weight the switch writes, a group workspace that
    overlaps a problem's y, and a bound output vector inside a weight are all
    refused on the host (DLM_EINVAL); nothing changes."""
    E, r = 4, 16
    W = (0.02 * torch.randn(64, 64, device="cuda")).bfloat16()
    A = (0.02 * torch.randn(E, r, 64, device="cuda")).bfloat16()
    B = (0.02 * torch.randn(E, 64, r, device="cuda")).bfloat16()
    W0 = W.clone()
    L = dlm.Layers([(W, A, B)], E, r, 1.0)
    inside = W.view(-1)[64:68].view(torch.int32)   # 8 bytes of W read as idx[2]
    g = torch.tensor([0.5, 0.5], device="cuda")
    with pytest.raises(dlm.DLMError) as e:
        L.switch(None, (inside, g))
    assert e.value.status == dlm.DLM_EINVAL
    ys = [W.view(-1)[:128].view(torch.float32)]     # 64 fp32 outputs inside W
    with pytest.raises(dlm.DLMError) as e:
        L.bind_vectors([torch.zeros(64, device="cuda").bfloat16()], ys)
    assert e.value.status == dlm.DLM_EINVAL
    torch.cuda.synchronize()
    assert torch.equal(W, W0)
    L.close()
    T = 40
    x = torch.randn(T, 64, device="cuda").bfloat16()
    y = torch.zeros(T, 64, device="cuda").bfloat16()
    grp = dlm.SgmmGroup([(x, A, B, y)], E, r, 1.0)
    n = dlm.sgmm_workspace_size(T, 64, E, r, 1)
    big = torch.zeros(n + T * 64 * 2 + 256, dtype=torch.uint8, device="cuda")
    ws_over_y = big[256:256 + n]
    idx = torch.zeros(T, 2, dtype=torch.int32, device="cuda")
    gg = torch.zeros(T, 2, device="cuda")
    grp2 = dlm.SgmmGroup([(x, A, B, big[:T * 64 * 2].view(torch.bfloat16).view(T, 64))], E, r, 1.0)
    with pytest.raises(dlm.DLMError) as e:
        grp2.run(idx, gg, workspace=ws_over_y)
    assert e.value.status == dlm.DLM_EINVAL
    grp.close()
    grp2.close()


def test_sgmm_without_workspace_raises_on_a_rejected_set():
    E, r, T = 4, 16, 8
    x = torch.randn(T, 64, device="cuda").bfloat16()
    A = (0.02 * torch.randn(E, r, 64, device="cuda")).bfloat16()
    B = (0.02 * torch.randn(E, 64, r, device="cuda")).bfloat16()
    y = torch.zeros(T, 64, device="cuda").bfloat16()
    idx = torch.zeros(T, 2, dtype=torch.int32, device="cuda")
    idx[3, 1] = E   # out of range
    g = torch.ones(T, 2, device="cuda")
    with pytest.raises(dlm.DLMError) as e:
        dlm.sgmm(x, idx, g, A, B, y, 1.0)
    assert e.value.status == dlm.DLM_EDEVICE
    assert (y == 0).all()
