"""dlm_sgmm_noalloc (the SGMM with its workspace in the library's static
scratch array) called through the C ABI gives bitwise the same y as dlm_sgmm
with a caller workspace, on two calls in a row on the same device, the second
with a smaller input; both are also held to the oracle.  Its status word
reports a rejected set, and a call larger than the scratch array is refused
before anything runs."""
import ctypes as C

import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth
from gpu_util import check_bf16

pytestmark = pytest.mark.gpu

SPLIT = 2.0 ** -16


def _inputs(T, d_in, d_out, E, r, key):
    dt = torch.bfloat16
    x = synth.normal_device((T, d_in), 1.0, dt, "cuda", "noalloc", key, "x")
    A = synth.normal_device((E, r, d_in), 0.02, dt, "cuda", "noalloc", key, "A")
    B = synth.normal_device((E, d_out, r), 0.02, dt, "cuda", "noalloc", key, "B")
    y = synth.normal_device((T, d_out), 0.02 * d_in ** 0.5, dt, "cuda", "noalloc", key, "y0")
    rng = np.random.default_rng(key)
    idx = np.stack([rng.choice(E, 2, replace=False) for _ in range(T)]).astype(np.int32)
    idx[rng.random(T) < 0.1, 1] = -1
    idx[rng.random(T) < 0.05] = -1
    g = rng.random((T, 2)).astype(np.float32)
    return x, A, B, y, torch.from_numpy(idx), torch.from_numpy(g)


def _call_noalloc(x, idx, g, A, B, y, scale, status):
    lib = dlm.load()
    T, d_in = x.shape
    E, r, _ = A.shape
    d_out = B.shape[1]
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.dlm_sgmm_noalloc(C.c_void_p(x.data_ptr()), C.c_void_p(idx.data_ptr()), C.c_void_p(g.data_ptr()),
                                C.c_void_p(A.data_ptr()), C.c_void_p(B.data_ptr()), C.c_void_p(y.data_ptr()),
                                T, d_in, d_out, E, r, C.c_float(scale), dlm.DLM_BF16,
                                None if status is None else C.c_void_p(status.data_ptr()), s)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    """Two calls in a row, the second smaller.  The first call on a device looks
    up the scratch array's device address, which is when the runtime places the
    array in that device's memory; no call after it changes free memory."""
    status = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    cases = [(3000, 1104, 520, 8, 16, 2.0, 1), (70, 264, 136, 16, 64, 1.0, 2)]
    for call, (T, d_in, d_out, E, r, scale, key) in enumerate(cases):
        print(f"[noalloc] T={T} d_in={d_in} d_out={d_out} E={E} r={r}", flush=True)
        x, A, B, y, idx, g = _inputs(T, d_in, d_out, E, r, key)
        y0 = y.clone()
        idx_d, g_d = idx.cuda(), g.cuda()
        y_ref = y0.clone()
        ws = dlm.sgmm_workspace(T, d_in, E, r)
        dlm.sgmm(x, idx_d, g_d, A, B, y_ref, scale, ws)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        rc = _call_noalloc(x, idx_d, g_d, A, B, y, scale, status)
        assert rc == dlm.DLM_OK, dlm.load().dlm_last_error()
        torch.cuda.synchronize()
        if call > 0:
            assert torch.cuda.mem_get_info()[0] == free0
        assert status.item() == 0
        assert dlm.sgmm_status(ws) == dlm.DLM_OK
        assert torch.equal(y, y_ref)
        ref, ex, ab = oracle.sgmm(x.cpu(), idx, g, A.cpu(), B.cpu(), y0.cpu(), scale, with_stats=True)
        check_bf16(y.cpu(), ref, ex, ab, d_in + 2 * r + 2, extra=SPLIT, what=f"noalloc T={T}")


def test_noalloc_status_and_size_limit():
    T, d_in, d_out, E, r = 40, 64, 64, 4, 16
    x, A, B, y, idx, g = _inputs(T, d_in, d_out, E, r, 3)
    y0 = y.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad = idx.clone()
    bad[7, 0] = E  # out of range: the call is a no-op on y and reports it
    assert _call_noalloc(x, bad.cuda(), g.cuda(), A, B, y, 1.0, status) == dlm.DLM_OK
    torch.cuda.synchronize()
    assert status.item() != 0
    assert torch.equal(y, y0)
    # a good call on the same scratch afterwards clears the word and works
    assert _call_noalloc(x, idx.cuda(), g.cuda(), A, B, y, 1.0, status) == dlm.DLM_OK
    torch.cuda.synchronize()
    assert status.item() == 0
    ref, ex, ab = oracle.sgmm(x.cpu(), idx, g, A.cpu(), B.cpu(), y0.cpu(), 1.0, with_stats=True)
    check_bf16(y.cpu(), ref, ex, ab, d_in + 2 * r + 2, extra=SPLIT, what="noalloc after a rejected set")
    # NULL status is allowed; repeated calls allocate nothing
    idx_d, g_d = idx.cuda(), g.cuda()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        assert _call_noalloc(x, idx_d, g_d, A, B, y, 1.0, None) == dlm.DLM_OK
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    # a workspace past the scratch array is refused on the host, nothing enqueued
    T2, d2 = 70000, 8192
    need = dlm.sgmm_workspace_size(T2, d2, 8, 128)
    assert need > 32 << 20
    xb = torch.empty((T2, d2), dtype=torch.bfloat16, device="cuda")
    Ab = torch.empty((8, 128, d2), dtype=torch.bfloat16, device="cuda")
    Bb = torch.empty((8, 8, 128), dtype=torch.bfloat16, device="cuda")
    yb = torch.empty((T2, 8), dtype=torch.bfloat16, device="cuda")
    ib = torch.full((T2, 2), -1, dtype=torch.int32, device="cuda")
    gb = torch.zeros((T2, 2), dtype=torch.float32, device="cuda")
    assert _call_noalloc(xb, ib, gb, Ab, Bb, yb, 1.0, status) == dlm.DLM_EWORKSPACE
