"""SGMM parity on small and ragged shapes, edge cases and the device error path.
Inputs are generated; the oracle recomputes every row in binary64."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import oracle
import synth
from gpu_util import check_bf16, check_f32

pytestmark = pytest.mark.gpu

# The expand feeds u = s*g*v to the MFMA as hi + lo bf16 terms: a relative
# representation error of at most 2^-17 per term on top of fp32 accumulation.
SPLIT = 2.0 ** -16


def _problem(T, d_in, d_out, E, r, dt, key):
    x = synth.normal_device((T, d_in), 1.0, dt, "cuda", key, "x")
    A = synth.normal_device((E, r, d_in), 0.02, dt, "cuda", key, "A")
    B = synth.normal_device((E, d_out, r), 0.02, dt, "cuda", key, "B")
    y = synth.normal_device((T, d_out), 0.02 * d_in ** 0.5, dt, "cuda", key, "y0")
    return x, A, B, y


def _sets(T, E, rng, p_empty=0.1, p_dup=0.05, p_none=0.05):
    idx = np.empty((T, 2), np.int32)
    for t in range(T):
        idx[t] = rng.choice(E, size=2, replace=E < 2)
        u = rng.random()
        if u < p_empty:
            idx[t, 1] = -1
        elif u < p_empty + p_dup:
            idx[t, 1] = idx[t, 0]
        elif u < p_empty + p_dup + p_none:
            idx[t] = -1
    g = rng.random((T, 2)).astype(np.float32)
    return torch.from_numpy(idx), torch.from_numpy(g)


def _check(x, idx, g, A, B, y0, y, scale, what):
    ref, ex, ab = oracle.sgmm(x.cpu(), idx.cpu(), g.cpu(), A.cpu(), B.cpu(), y0, scale,
                              with_stats=True)
    d_in, r = x.shape[1], A.shape[1]
    n = d_in + 2 * r + 2
    if y.dtype == torch.float32:
        return check_f32(y.cpu(), ex, ab, n, what)
    return check_bf16(y.cpu(), ref, ex, ab, n, extra=SPLIT, what=what)


CASES = [
    # (T, d_in, d_out, E, r, scale, dtype)
    (16, 64, 64, 4, 4, 1.0, torch.float32),          # tiny fp32 workload shape
    (33, 96, 40, 3, 5, 2.0, torch.float32),
    (1, 64, 64, 8, 16, 1.0, torch.bfloat16),
    (2, 4104, 1032, 8, 16, 1.0, torch.bfloat16),     # few rows (one launch), a ragged last column group
    (3, 200, 264, 8, 4, 2.0, torch.bfloat16),        # few rows, r < 16 and r % 8 != 0
    (4, 520, 40, 3, 100, 0.5, torch.bfloat16),       # few rows, rank 100
    (4, 64, 2056, 32, 128, 1.0, torch.bfloat16),     # few rows, largest rank and expert count
    (5, 200, 264, 8, 16, 2.0, torch.bfloat16),       # ragged everything
    (33, 64, 72, 2, 16, 1.0, torch.bfloat16),
    (100, 136, 520, 8, 4, 1.0, torch.bfloat16),      # r < 16, r % 8 != 0
    (64, 128, 256, 8, 24, 1.0, torch.bfloat16),
    (70, 72, 64, 16, 64, 1.0, torch.bfloat16),       # 70B rank, many experts
    (40, 64, 64, 32, 16, 1.0, torch.bfloat16),       # most experts
    (2500, 64, 64, 32, 16, 1.0, torch.bfloat16),     # most experts, waves with many distinct pairs
    (20, 64, 96, 4, 128, 0.5, torch.bfloat16),       # largest rank
    (50, 200, 96, 4, 40, 1.0, torch.bfloat16),       # rank 40 (3 rank chunks)
    (40, 136, 72, 4, 80, 1.0, torch.bfloat16),       # rank 80 (5)
    (33, 64, 64, 2, 96, 1.0, torch.bfloat16),        # rank 96 (6)
    (20, 520, 40, 3, 100, 0.5, torch.bfloat16),      # rank 100 (7): r % 8 != 0, two LDS steps
    (300, 256, 264, 8, 16, 1.0, torch.bfloat16),
    (40, 2056, 72, 8, 16, 1.0, torch.bfloat16),      # two K slices of 2048, the last 8 wide
    (40, 4104, 72, 8, 16, 1.0, torch.bfloat16),      # three K slices, 4 + 4 + 1 LDS steps
    (70, 1096, 136, 16, 64, 0.5, torch.bfloat16),    # three LDS steps, rounds of N blocks per tile
    (70, 4616, 136, 16, 64, 0.5, torch.bfloat16),    # rounds of N blocks over three K slices
    (40, 4104, 72, 4, 80, 1.0, torch.bfloat16),      # rank 80 over three K slices: the K-slice sum launch
    (60, 4104, 200, 8, 24, 1.0, torch.bfloat16),     # two rank chunks, three K slices added by the expand
    (70, 2568, 520, 16, 32, 1.0, torch.bfloat16),    # two whole rank chunks, two K slices
    (45, 6152, 136, 4, 40, 0.5, torch.bfloat16),     # three rank chunks (r % 16 != 0), four K slices
    (33, 4608, 64, 8, 48, 2.0, torch.bfloat16),      # three whole rank chunks, three K slices
    (36, 2056, 1096, 3, 128, 0.5, torch.bfloat16),   # largest rank over two K slices, a ragged column group
    (100, 1024, 64, 8, 128, 1.0, torch.bfloat16),    # two whole LDS steps, largest rank
    (9, 2100, 24, 4, 8, 1.0, torch.float32),         # fp32 past one slice width
    (9000, 64, 72, 8, 16, 1.0, torch.bfloat16),      # more rows than the segment's LDS caches
    (3000, 72, 40, 4, 8, 1.0, torch.float32),        # fp32, one segmentation launch over three chunks
    (12, 64, 64, 1, 16, 1.0, torch.bfloat16),         # one expert: every used slot is expert 0
    (7, 8, 8, 2, 1, 1.0, torch.bfloat16),             # rank 1, one 8-wide chunk of d_in
    (3, 16, 8, 1, 1, 3.0, torch.float32),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_sgmm_parity(ci):
    T, d_in, d_out, E, r, scale, dt = CASES[ci]
    print(f"[sgmm] case {ci}: T={T} d_in={d_in} d_out={d_out} E={E} r={r} {dt}", flush=True)
    x, A, B, y = _problem(T, d_in, d_out, E, r, dt, 3000 + ci)
    idx, g = _sets(T, E, np.random.default_rng(ci))
    y0 = y.cpu().clone()
    idx_d, g_d = idx.cuda(), g.cuda()
    ws = dlm.sgmm_workspace(T, d_in, E, r)
    dlm.sgmm(x, idx_d, g_d, A, B, y, scale, ws)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    st = _check(x, idx, g, A, B, y0, y, scale, f"sgmm case {ci}")
    print(st, flush=True)
    # rows whose two slots are empty are not touched
    none = (idx == -1).all(1)
    assert torch.equal(y.cpu()[none], y0[none])


def test_sgmm_zero_gates_and_slot_swap():
    T, d_in, d_out, E, r = 48, 128, 136, 8, 16
    x, A, B, y = _problem(T, d_in, d_out, E, r, torch.bfloat16, 3100)
    idx, g = _sets(T, E, np.random.default_rng(5), 0, 0, 0)
    y0 = y.clone()
    ws = dlm.sgmm_workspace(T, d_in, E, r)
    dlm.sgmm(x, idx.cuda(), torch.zeros_like(g).cuda(), A, B, y, 1.0, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    y1 = y0.clone()
    dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y1, 1.0, ws)
    y2 = y0.clone()
    dlm.sgmm(x, idx.flip(1).contiguous().cuda(), g.flip(1).contiguous().cuda(), A, B, y2, 1.0, ws)
    torch.cuda.synchronize()
    # with the slots swapped a row keeps its pair, hence its tile and union: same bits
    assert torch.equal(y1, y2)


def test_sgmm_single_set_matches_gemm_reference():
    """All rows on one set: y + s(g0 X A0^T B0^T + g1 X A1^T B1^T), a plain GEMM chain (fp32 CPU)."""
    T, d_in, d_out, E, r = 96, 256, 192, 8, 16
    x, A, B, y = _problem(T, d_in, d_out, E, r, torch.bfloat16, 3101)
    y0 = y.cpu().clone()
    idx = torch.tensor([[2, 6]] * T, dtype=torch.int32)
    g = torch.tensor([[0.75, 0.25]] * T, dtype=torch.float32)
    dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y, 2.0)
    torch.cuda.synchronize()
    X, Ad, Bd = x.cpu().double(), A.cpu().double(), B.cpu().double()
    ref = y0.double() + 2.0 * (0.75 * (X @ Ad[2].T) @ Bd[2].T + 0.25 * (X @ Ad[6].T) @ Bd[6].T)
    assert (y.cpu().double() - ref).abs().max().item() < 0.02
    _check(x, idx, g, A, B, y0, y, 2.0, "single set")


@pytest.mark.parametrize("T,bads", [
    (40, [((7, 0), 4), ((3, 1), -2), ((20, 0), None)]),
    # one segmentation launch over three chunks: the bad row in another chunk
    # than most workgroups' own
    (3000, [((2990, 0), 4), ((5, 1), -2), ((1500, 0), None)]),
    # count launch first (more than 8192 rows)
    (9000, [((8500, 1), 4), ((100, 0), None)]),
])
def test_sgmm_bad_set_is_a_noop_with_status(T, bads):
    d_in, d_out, E, r = 64, 64, 4, 16
    print(f"[sgmm] bad sets T={T}", flush=True)
    x, A, B, y = _problem(T, d_in, d_out, E, r, torch.bfloat16, 3102)
    y0 = y.clone()
    idx, g = _sets(T, E, np.random.default_rng(9), 0, 0, 0)
    ws = dlm.sgmm_workspace(T, d_in, E, r)
    for bad_i, bad_g in bads:
        ii, gg = idx.clone(), g.clone()
        if bad_g is None:
            gg[bad_i] = float("nan")
        else:
            ii[bad_i] = bad_g
        dlm.sgmm(x, ii.cuda(), gg.cuda(), A, B, y, 1.0, ws)
        assert dlm.sgmm_status(ws) == dlm.DLM_EDEVICE
        assert torch.equal(y, y0)
    # the status word was cleared; a good call works again on the same workspace
    dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y, 1.0, ws)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    _check(x, idx, g, A, B, y0.cpu(), y, 1.0, "after bad set")


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_sgmm_few_rows_single_launch(T):
    """Calls with at most four rows skip the segmentation: every row form --
    two experts, one slot empty, the same expert twice, both slots empty --
    against the oracle on three problems of different shapes, each run alone
    (one launch) and all three as a group (two launches); a rejected set
    leaves y untouched and sets the status word, alone and in a group."""
    E, r = 8, 16
    shapes = [(4104, 1032), (200, 264), (11008, 4096)]
    print(f"[sgmm] few rows T={T}", flush=True)
    probs = [_problem(T, i, o, E, r, torch.bfloat16, 3400 + 10 * T + k) for k, (i, o) in enumerate(shapes)]
    idx = torch.tensor([[1, 5], [2, -1], [3, 3], [-1, -1]][:T], dtype=torch.int32)
    g = torch.tensor([[0.7, 0.3], [1.0, 0.5], [0.6, 0.4], [0.5, 0.5]][:T], dtype=torch.float32)
    assert dlm.sgmm_launches(T, 11008, r) == 1 and dlm.sgmm_launches(T, 11008, r, 3) == 2
    y0s = [p[3].clone() for p in probs]
    grp = dlm.SgmmGroup(probs, E, r, 2.0)
    ws = grp.run(idx.cuda(), g.cuda())
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    none = (idx == -1).all(1)
    for k, (x, A, B, y) in enumerate(probs):
        _check(x, idx, g, A, B, y0s[k].cpu(), y, 2.0, f"few rows T={T} problem {k}")
        assert torch.equal(y.cpu()[none], y0s[k].cpu()[none])
        y1 = y0s[k].clone()
        dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y1, 2.0)
        _check(x, idx, g, A, B, y0s[k].cpu(), y1, 2.0, f"few rows T={T} problem {k} alone")
        assert torch.equal(y1.cpu()[none], y0s[k].cpu()[none])
    bad = idx.clone()
    bad[0, 0] = E
    x0, A0, B0, _ = probs[0]
    y2 = y0s[0].clone()
    ws1 = dlm.sgmm_workspace(T, shapes[0][0], E, r)
    dlm.sgmm(x0, bad.cuda(), g.cuda(), A0, B0, y2, 2.0, ws1)
    assert dlm.sgmm_status(ws1) == dlm.DLM_EDEVICE
    assert torch.equal(y2, y0s[0])
    before = [p[3].clone() for p in probs]
    ws = grp.run(bad.cuda(), g.cuda())
    assert dlm.sgmm_status(ws) == dlm.DLM_EDEVICE
    assert all(torch.equal(p[3], b) for p, b in zip(probs, before))
    grp.close()


@pytest.mark.parametrize("r,shapes", [
    (16, [(64, 128), (200, 64), (96, 264)]),
    # several K slices per problem (the expand adds them), different counts per problem
    (24, [(4104, 136), (2056, 64), (96, 1040)]),
])
def test_sgmm_group_matches_single_calls(r, shapes):
    T, E = 50, 8
    probs = [_problem(T, i, o, E, r, torch.bfloat16, 3200 + k) for k, (i, o) in enumerate(shapes)]
    idx, g = _sets(T, E, np.random.default_rng(11))
    y0s = [p[3].clone() for p in probs]
    grp = dlm.SgmmGroup(probs, E, r, 2.0)
    grp.run(idx.cuda(), g.cuda())
    torch.cuda.synchronize()
    for k, (x, A, B, y) in enumerate(probs):
        y1 = y0s[k].clone()
        dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y1, 2.0)
        torch.cuda.synchronize()
        assert torch.equal(y1, y), k
        _check(x, idx, g, A, B, y0s[k].cpu(), y, 2.0, f"group problem {k}")


def test_sgmm_group_shared_bank_and_repack():
    """Two problems on one A bank (one packed copy), three K slices; after A is
    changed in place, repack makes the next run use the new values."""
    T, E, r = 70, 8, 16
    x1, A, B1, y1 = _problem(T, 2056, 64, E, r, torch.bfloat16, 3300)
    x2, _, B2, y2 = _problem(T, 2056, 136, E, r, torch.bfloat16, 3301)
    idx, g = _sets(T, E, np.random.default_rng(12))
    y10, y20 = y1.cpu().clone(), y2.cpu().clone()
    grp = dlm.SgmmGroup([(x1, A, B1, y1), (x2, A, B2, y2)], E, r, 1.0)
    grp.run(idx.cuda(), g.cuda())
    torch.cuda.synchronize()
    _check(x1, idx, g, A, B1, y10, y1, 1.0, "shared bank, problem 0")
    _check(x2, idx, g, A, B2, y20, y2, 1.0, "shared bank, problem 1")
    A.mul_(-0.5)  # exact in bf16
    y1.copy_(y10)
    y2.copy_(y20)
    grp.repack()
    grp.run(idx.cuda(), g.cuda())
    torch.cuda.synchronize()
    _check(x1, idx, g, A, B1, y10, y1, 1.0, "repacked, problem 0")
    _check(x2, idx, g, A, B2, y20, y2, 1.0, "repacked, problem 1")
    grp.close()


def test_sgmm_all_rows_released_leaves_y_bitwise():
    T, d_in, d_out, E, r = 64, 256, 136, 8, 16
    x, A, B, y = _problem(T, d_in, d_out, E, r, torch.bfloat16, 3300)
    y0 = y.clone()
    idx = torch.full((T, 2), -1, dtype=torch.int32, device="cuda")
    g = torch.zeros((T, 2), dtype=torch.float32, device="cuda")
    ws = dlm.sgmm_workspace(T, d_in, E, r)
    dlm.sgmm(x, idx, g, A, B, y, 1.0, ws)
    torch.cuda.synchronize()
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    assert torch.equal(y, y0)


def test_sgmm_empty_batch_is_noop():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(4, 16, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(4, 64, 16, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(0, 2, dtype=torch.int32, device="cuda")
    g = torch.empty(0, 2, dtype=torch.float32, device="cuda")
    dlm.sgmm(x, idx, g, A, B, y, 1.0)
    torch.cuda.synchronize()


def _host_segmentation(idx: np.ndarray, E: int):
    """Rows ordered by their unordered expert pair, stably (row order within a
    pair); rows with two empty slots left out.  Returns (perm, pair keys)."""
    a = np.minimum(idx[:, 0], idx[:, 1]).astype(np.int64)
    b = np.maximum(idx[:, 0], idx[:, 1]).astype(np.int64)
    key = (a + 1) * (E + 1) + (b + 1)
    live = np.flatnonzero(b >= 0)
    order = live[np.argsort(key[live], kind="stable")]
    return order.astype(np.int32), key


@pytest.mark.parametrize("T,E,seed", [(9000, 8, 1), (4096, 8, 2), (2500, 32, 3), (1500, 4, 4), (1025, 2, 5),
                                      (8192, 16, 6), (8193, 3, 7)])
def test_segment_order_equals_host_stable_sort(T, E, seed):
    """The row order the segmentation writes (the workspace's perm list, after
    the 256-byte header) is the stable sort of the rows by unordered pair, bit
    for bit; positions past the live rows hold -1; the header counts match.
    Covers batches past the first 1024 rows and past the 8192-row key cache."""
    print(f"[sgmm] segment T={T} E={E}", flush=True)
    d_in = d_out = 64
    x, A, B, y = _problem(T, d_in, d_out, E, 16, torch.bfloat16, 3400 + seed)
    idx, g = _sets(T, E, np.random.default_rng(100 + seed))
    ws = dlm.sgmm_workspace(T, d_in, E, 16)
    dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, y, 1.0, ws)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    T_pad = (T + 31) // 32 * 32
    w = ws.cpu()
    hdr = w[:256].view(torch.int32).numpy()
    perm = w[256:256 + 4 * T_pad].view(torch.int32).numpy()
    want, _ = _host_segmentation(idx.numpy(), E)
    n_pos = len(want)
    assert hdr[1] == n_pos and hdr[2] == (n_pos + 31) // 32
    assert np.array_equal(perm[:n_pos], want)
    assert (perm[n_pos:] == -1).all()


@pytest.mark.parametrize("T,d_in,d_out,E,r,seed", [(64, 4104, 520, 8, 16, 1), (37, 200, 72, 16, 40, 2),
                                                   (64, 136, 64, 4, 128, 3), (6, 64, 1096, 2, 24, 4)])
def test_inline_row_order_equals_the_segmentation(T, d_in, d_out, E, r, seed):
    """Up to 64 rows (and fewer than 256 (problem, tile) pairs) the shrink and
    expand order the rows themselves (no segmentation launch).  The same rows
    followed by released rows up to 65 (the segmentation launch runs, and
    released rows take no position) must give bitwise the same y for the first
    T rows, leave the released rows alone, and agree with the oracle; the
    header words the shrink publishes match the segmentation's."""
    print(f"[sgmm] inline order T={T} d_in={d_in} r={r}", flush=True)
    T2 = 65
    x, A, B, y = _problem(T2, d_in, d_out, E, r, torch.bfloat16, 3600 + seed)
    idx, g = _sets(T2, E, np.random.default_rng(200 + seed))
    idx[T:] = -1
    assert dlm.sgmm_launches(T, d_in, r) == 2 and dlm.sgmm_launches(T2, d_in, r) == 3
    y0 = y.clone()
    ya, yb = y[:T].clone(), y.clone()
    ws = dlm.sgmm_workspace(T2, d_in, E, r)
    dlm.sgmm(x[:T].contiguous(), idx[:T].contiguous().cuda(), g[:T].contiguous().cuda(), A, B, ya, 1.0, ws)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    hdr_a = ws[:256].cpu().view(torch.int32).numpy()[:3].copy()
    dlm.sgmm(x, idx.cuda(), g.cuda(), A, B, yb, 1.0, ws)
    assert dlm.sgmm_status(ws) == dlm.DLM_OK
    hdr_b = ws[:256].cpu().view(torch.int32).numpy()[:3].copy()
    assert np.array_equal(hdr_a, hdr_b), (hdr_a, hdr_b)
    assert torch.equal(ya, yb[:T]), "inline order differs from the segmentation"
    assert torch.equal(yb[T:], y0[T:]), "a released row was written"
    _check(x[:T], idx[:T], g[:T], A, B, y0[:T].cpu(), ya, 1.0, f"inline order T={T}")
