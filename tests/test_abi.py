"""C-ABI library checks that need no GPU: it loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call
(every call below fails validation, so no device memory is ever touched)."""
import ctypes as C
import os

import pytest

import dynamic_lora_moe_amd as dlm

pytestmark = pytest.mark.skipif(not os.path.exists(dlm.LIB_PATH), reason="libdlm.so not built")

FAKE = 0x100000  # a 256-byte aligned address that validation rejects before use


@pytest.fixture(scope="module")
def lib():
    return dlm.load()


def test_exports_every_header_function(lib):
    names = dlm.header_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dlm.h but not exported"
    assert lib.dlm_version().decode().startswith("dlm")


def test_header_status_codes_match_binding():
    text = open(dlm.HEADER).read()
    for name, val in [("DLM_OK", 0), ("DLM_EINVAL", -1), ("DLM_ESHAPE", -2), ("DLM_EDTYPE", -3),
                      ("DLM_EALIGN", -4), ("DLM_EWORKSPACE", -5), ("DLM_EHIP", -6),
                      ("DLM_EDEVICE", -7), ("DLM_ENOMEM", -8)]:
        assert f"{name} = {val}" in text
        assert dlm.STATUS_NAMES[val] == name


def _err(lib):
    return lib.dlm_last_error().decode()


def test_pregate_validation(lib):
    P = C.c_void_p
    assert lib.dlm_pregate(P(FAKE), P(FAKE), 4, 64, 1, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert "E=1" in _err(lib)
    assert lib.dlm_pregate(P(FAKE), P(FAKE), 4, 64, 33, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert lib.dlm_pregate(P(FAKE), P(FAKE), 4, 0, 8, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert lib.dlm_pregate(P(FAKE), P(FAKE), -1, 64, 8, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert lib.dlm_pregate(P(FAKE), P(FAKE), 4, 64, 8, 7, P(FAKE), P(FAKE), None) == dlm.DLM_EDTYPE
    assert lib.dlm_pregate(None, P(FAKE), 4, 64, 8, 1, P(FAKE), P(FAKE), None) == dlm.DLM_EINVAL
    assert lib.dlm_pregate(P(FAKE), P(FAKE), 4, 64, 8, 1, None, P(FAKE), None) == dlm.DLM_EINVAL
    # T = 0 is a valid no-op that touches nothing
    assert lib.dlm_pregate(None, None, 0, 64, 8, 1, None, None, None) == dlm.DLM_OK


def _projs(*ps):
    arr = (dlm.dlm_proj * len(ps))()
    for i, p in enumerate(ps):
        arr[i] = dlm.dlm_proj(*p)
    return arr


def test_layers_create_validation(lib):
    h = C.c_void_p()
    ok = (FAKE, FAKE, FAKE, 64, 64)
    assert lib.dlm_layers_create(None, 1, 4, 4, 1.0, 1, C.byref(h)) == dlm.DLM_EINVAL
    assert lib.dlm_layers_create(_projs(ok), 1, 4, 4, 1.0, 1, None) == dlm.DLM_EINVAL
    assert lib.dlm_layers_create(_projs(ok), 0, 4, 4, 1.0, 1, C.byref(h)) == dlm.DLM_EINVAL
    assert lib.dlm_layers_create(_projs(ok), 1, 0, 4, 1.0, 1, C.byref(h)) == dlm.DLM_ESHAPE
    assert lib.dlm_layers_create(_projs(ok), 1, 33, 4, 1.0, 1, C.byref(h)) == dlm.DLM_ESHAPE
    assert lib.dlm_layers_create(_projs(ok), 1, 4, 0, 1.0, 1, C.byref(h)) == dlm.DLM_ESHAPE
    assert lib.dlm_layers_create(_projs(ok), 1, 4, 129, 1.0, 1, C.byref(h)) == dlm.DLM_ESHAPE
    assert lib.dlm_layers_create(_projs(ok), 1, 4, 4, 1.0, 5, C.byref(h)) == dlm.DLM_EDTYPE
    assert lib.dlm_layers_create(_projs(ok), 1, 4, 4, float("nan"), 1, C.byref(h)) == dlm.DLM_EINVAL
    assert lib.dlm_layers_create(_projs((0, FAKE, FAKE, 64, 64)), 1, 4, 4, 1.0, 1, C.byref(h)) == dlm.DLM_EINVAL
    assert lib.dlm_layers_create(_projs((FAKE, FAKE, FAKE, 0, 64)), 1, 4, 4, 1.0, 1, C.byref(h)) == dlm.DLM_ESHAPE
    # bf16 fast path needs 16-byte aligned pointers and d_in % 8 == 0; the second
    # weight of the list is the bad one, so the error names it
    assert lib.dlm_layers_create(_projs(ok, (FAKE + 2, FAKE, FAKE, 64, 64)), 2, 4, 4, 1.0, 1,
                                 C.byref(h)) == dlm.DLM_EALIGN
    assert "proj 1" in _err(lib)
    assert lib.dlm_layers_create(_projs((FAKE, FAKE, FAKE, 64, 60)), 1, 4, 4, 1.0, 1, C.byref(h)) == dlm.DLM_EALIGN
    assert h.value is None


def test_switch_and_status_validation(lib):
    P = C.c_void_p
    assert lib.dlm_switch(None, None, None, None, None, None) == dlm.DLM_EINVAL
    assert lib.dlm_layers_destroy(None) == dlm.DLM_EINVAL
    assert lib.dlm_layers_status(None, None, None) == dlm.DLM_EINVAL
    assert lib.dlm_switch_launches(None) == 0
    assert lib.dlm_sgmm_status(None, None, None) == dlm.DLM_EINVAL
    assert lib.dlm_sgmm_group_destroy(None) == dlm.DLM_EINVAL
    assert lib.dlm_sgmm_group_run(None, P(FAKE), P(FAKE), 4, P(FAKE), 1 << 20, None) == dlm.DLM_EINVAL


def test_centroid_pregate_validation(lib):
    P = C.c_void_p
    f = lib.dlm_pregate_centroid
    assert f(P(FAKE), P(FAKE), 4, 64, 0, 2, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert "E=0" in _err(lib)
    assert f(P(FAKE), P(FAKE), 4, 64, 33, 2, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert f(P(FAKE), P(FAKE), 4, 64, 8, 0, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert f(P(FAKE), P(FAKE), 4, 64, 8, 1025, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert f(P(FAKE), P(FAKE), 4, 0, 8, 2, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert f(P(FAKE), P(FAKE), -1, 64, 8, 2, 1, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
    assert f(P(FAKE), P(FAKE), 4, 64, 8, 2, 5, P(FAKE), P(FAKE), None) == dlm.DLM_EDTYPE
    assert f(P(FAKE), None, 4, 64, 8, 2, 1, P(FAKE), P(FAKE), None) == dlm.DLM_EINVAL
    # E = 1 is valid here (a single adapter always wins); T = 0 touches nothing
    assert f(None, None, 0, 64, 1, 1, 1, None, None, None) == dlm.DLM_OK


def test_product_entry_points_validation(lib):
    P = C.c_void_p
    assert lib.dlm_layers_bind_vectors(None, P(FAKE), P(FAKE)) == dlm.DLM_EINVAL
    assert lib.dlm_gemv(None, None) == dlm.DLM_EINVAL
    assert lib.dlm_switch_gemv(None, None, None, None, None, None) == dlm.DLM_EINVAL
    assert lib.dlm_switch_gemv_launches(None) == 0
    assert lib.dlm_gemv_unmerged(None, None, None, None) == dlm.DLM_EINVAL
    assert lib.dlm_gemv_unmerged_launches(None) == 0
    assert lib.dlm_layers_repack(None, None) == dlm.DLM_EINVAL


def test_sgmm_launch_count(lib):
    f = lib.dlm_sgmm_launches
    assert f(0, 4096, 16, 1, dlm.DLM_BF16) == 0
    # up to 4 rows: one launch for one problem, two for a group
    assert f(1, 4096, 16, 1, dlm.DLM_BF16) == 1
    assert f(4, 11008, 64, 1, dlm.DLM_BF16) == 1
    assert f(1, 4096, 128, 7, dlm.DLM_BF16) == 2
    # 5..64 rows and fewer than 256 (problem, tile) pairs: the shrink and
    # expand order the rows themselves (no segmentation launch) unless a
    # K-slice sum launch is needed
    assert f(5, 4096, 16, 1, dlm.DLM_BF16) == 2
    assert f(64, 11008, 64, 7, dlm.DLM_BF16) == 2
    assert f(64, 2048, 128, 1, dlm.DLM_BF16) == 2
    # segment, shrink, expand below 256 pairs; from 256 pairs up to rank 64 the
    # segmentation and one launch for the shrink and expand
    assert f(65, 4096, 16, 1, dlm.DLM_BF16) == 3
    assert f(1024, 4096, 64, 7, dlm.DLM_BF16) == 3
    assert f(1024, 4096, 64, 8, dlm.DLM_BF16) == 2
    assert f(64, 4096, 16, 128, dlm.DLM_BF16) == 2
    assert f(64, 4096, 16, 127, dlm.DLM_BF16) == 2
    # above rank 64 a K-slice sum launch runs when there are several slices
    assert f(64, 4096, 65, 1, dlm.DLM_BF16) == 4
    assert f(65, 2048, 128, 1, dlm.DLM_BF16) == 3
    assert f(64, 2049, 128, 1, dlm.DLM_BF16) == 4
    # one segmentation launch up to 8192 rows, a count launch before the
    # placement above
    assert f(8192, 4096, 16, 1, dlm.DLM_BF16) == 2
    assert f(8193, 4096, 16, 1, dlm.DLM_BF16) == 3
    assert f(8193, 4096, 80, 1, dlm.DLM_BF16) == 5
    assert f(1, 64, 16, 1, dlm.DLM_F32) == 3
    assert f(4096, 64, 16, 1, dlm.DLM_F32) == 3
    assert f(8193, 64, 16, 1, dlm.DLM_F32) == 4
    assert f(-1, 64, 16, 1, dlm.DLM_BF16) == -1 and "sgmm_launches" in _err(lib)
    assert f(4, 0, 16, 1, dlm.DLM_BF16) == -1
    assert f(4, 64, 0, 1, dlm.DLM_BF16) == -1
    assert f(4, 64, 129, 1, dlm.DLM_BF16) == -1
    assert f(4, 64, 16, 0, dlm.DLM_BF16) == -1
    assert f(4, 64, 16, 1, 7) == -1
    assert dlm.sgmm_launches(1, 11008, 16) == 1
    assert dlm.sgmm_launches(1, 11008, 16, 7) == 2
    assert dlm.sgmm_launches(64, 11008, 16) == 2
    assert dlm.sgmm_launches(65, 11008, 16) == 3
    assert dlm.sgmm_launches(64, 11008, 128) == 4


def test_sgmm_workspace_size(lib):
    b = C.c_size_t(0)
    assert lib.dlm_sgmm_workspace_size(4096, 11008, 8, 16, 7, C.byref(b)) == dlm.DLM_OK
    # the shrink's partial results dominate: 7 problems x 6 K slices of 2048 x
    # 4096 rows x 2 slots x 16 x 4 bytes
    assert b.value >= 7 * 6 * 4096 * 2 * 16 * 4
    assert b.value % 256 == 0
    one = C.c_size_t(0)
    assert lib.dlm_sgmm_workspace_size(4096, 1024, 8, 16, 7, C.byref(one)) == dlm.DLM_OK
    assert one.value < b.value
    small = C.c_size_t(0)
    assert lib.dlm_sgmm_workspace_size(64, 1024, 8, 16, 1, C.byref(small)) == dlm.DLM_OK
    assert small.value < one.value
    assert lib.dlm_sgmm_workspace_size(-1, 64, 8, 16, 1, C.byref(b)) == dlm.DLM_ESHAPE
    assert lib.dlm_sgmm_workspace_size(64, 0, 8, 16, 1, C.byref(b)) == dlm.DLM_ESHAPE
    assert lib.dlm_sgmm_workspace_size(64, 64, 0, 16, 1, C.byref(b)) == dlm.DLM_ESHAPE
    assert lib.dlm_sgmm_workspace_size(64, 64, 8, 0, 1, C.byref(b)) == dlm.DLM_ESHAPE
    assert lib.dlm_sgmm_workspace_size(64, 64, 8, 16, 0, C.byref(b)) == dlm.DLM_EINVAL
    assert lib.dlm_sgmm_workspace_size(64, 64, 8, 16, 1, None) == dlm.DLM_EINVAL


MB = 1 << 20


def test_sgmm_validation(lib):
    P = C.c_void_p
    ws = C.c_size_t(0)
    lib.dlm_sgmm_workspace_size(16, 64, 4, 16, 1, C.byref(ws))
    # every buffer at its own (fake) address, megabytes apart
    X, Y, IDX, G, A, B, W = (FAKE + k * MB for k in range(7))

    def call(x=X, idx=IDX, g=G, A=A, B=B, y=Y, T=16, d_in=64, d_out=64, E=4, r=16,
             s=1.0, dt=1, w=W, nb=ws.value):
        return lib.dlm_sgmm(P(x), P(idx), P(g), P(A), P(B), P(y), T, d_in, d_out, E, r, s, dt,
                            P(w), nb, None)

    assert call(T=-1) == dlm.DLM_ESHAPE
    assert call(E=0) == dlm.DLM_ESHAPE
    assert call(r=200) == dlm.DLM_ESHAPE
    assert call(dt=3) == dlm.DLM_EDTYPE
    assert call(s=float("inf")) == dlm.DLM_EINVAL
    assert call(x=0) == dlm.DLM_EINVAL
    assert call(idx=0) == dlm.DLM_EINVAL
    assert call(d_in=0) == dlm.DLM_ESHAPE
    assert call(d_out=60) == dlm.DLM_EALIGN
    assert call(A=FAKE + 8) == dlm.DLM_EALIGN
    assert call(y=X + 64) == dlm.DLM_EINVAL          # y overlaps x
    assert "overlap" in _err(lib)
    assert call(y=A + 512) == dlm.DLM_EINVAL         # y overlaps the A bank
    assert call(y=IDX - 1024) == dlm.DLM_EINVAL      # y runs into the sets
    assert call(w=Y + 256) == dlm.DLM_EINVAL         # the workspace overlaps y
    assert "workspace" in _err(lib)
    assert call(w=0) == dlm.DLM_EWORKSPACE
    assert call(nb=ws.value - 1) == dlm.DLM_EWORKSPACE
    assert call(w=W + 16) == dlm.DLM_EALIGN          # workspace must be 256-byte aligned
    assert call(T=0) == dlm.DLM_OK                   # nothing to do, nothing touched


def test_layers_create_refuses_aliased_buffers(lib):
    """A weight the switch writes in place may overlap no other weight and no
    bank (other weights' banks included); banks may share memory (read only)."""
    h = C.c_void_p()
    W0, W1, A0, B0 = FAKE, FAKE + MB, FAKE + 2 * MB, FAKE + 3 * MB
    # same weight twice
    assert lib.dlm_layers_create(_projs((W0, A0, B0, 64, 64), (W0, A0, B0, 64, 64)), 2, 4, 4, 1.0, 1,
                                 C.byref(h)) == dlm.DLM_EINVAL
    assert "overlaps" in _err(lib)
    # a weight running into another weight's bank
    assert lib.dlm_layers_create(_projs((W0, A0, B0, 64, 64), (A0 - 4096, A0 + 8192, B0, 64, 64)), 2, 4, 4,
                                 1.0, 1, C.byref(h)) == dlm.DLM_EINVAL
    # a weight inside its own B bank
    assert lib.dlm_layers_create(_projs((B0 + 256, A0, B0, 64, 64)), 1, 4, 4, 1.0, 1, C.byref(h)) == dlm.DLM_EINVAL
    assert h.value is None


def test_sgmm_noalloc_validation(lib):
    P = C.c_void_p
    X, Y, IDX, G, A, B, S = (FAKE + k * MB for k in range(7))

    def call(x=X, idx=IDX, g=G, A=A, B=B, y=Y, T=16, d_in=64, d_out=64, E=4, r=16, s=1.0, dt=1, st=S):
        return lib.dlm_sgmm_noalloc(P(x), P(idx), P(g), P(A), P(B), P(y), T, d_in, d_out, E, r, s, dt, P(st),
                                    None)

    assert call(E=0) == dlm.DLM_ESHAPE
    assert call(dt=3) == dlm.DLM_EDTYPE
    assert call(x=0) == dlm.DLM_EINVAL
    assert call(d_out=60) == dlm.DLM_EALIGN
    assert call(y=X + 64) == dlm.DLM_EINVAL
    assert call(st=Y + 4) == dlm.DLM_EINVAL          # the status word inside y
    # more scratch than the library's array holds: refused before anything runs
    assert call(T=70000, d_in=8192, r=128, E=8, y=1 << 40, idx=1 << 41, g=1 << 42, A=1 << 43, B=1 << 44,
                st=1 << 45) == dlm.DLM_EWORKSPACE
    assert "maximum" in _err(lib)
    assert call(T=0) == dlm.DLM_OK


def test_sgmm_group_create_validation(lib):
    h = C.c_void_p()
    arr = (dlm.dlm_sgmm_problem * 2)()
    arr[0] = dlm.dlm_sgmm_problem(FAKE, FAKE, FAKE, FAKE + (1 << 20), 64, 64)
    arr[1] = dlm.dlm_sgmm_problem(FAKE, FAKE, FAKE, FAKE + (1 << 20), 64, 12)
    assert lib.dlm_sgmm_group_create(None, 1, 4, 16, 1.0, 1, C.byref(h)) == dlm.DLM_EINVAL
    assert lib.dlm_sgmm_group_create(arr, 0, 4, 16, 1.0, 1, C.byref(h)) == dlm.DLM_EINVAL
    assert lib.dlm_sgmm_group_create(arr, 2, 4, 16, 1.0, 1, None) == dlm.DLM_EINVAL
    assert lib.dlm_sgmm_group_create(arr, 2, 40, 16, 1.0, 1, C.byref(h)) == dlm.DLM_ESHAPE
    # problem 1 has d_out = 12 (not a multiple of 8) for bf16
    assert lib.dlm_sgmm_group_create(arr, 2, 4, 16, 1.0, 1, C.byref(h)) == dlm.DLM_EALIGN
    assert "problem 1" in _err(lib)
    assert h.value is None


def test_grids_past_32_bits_are_refused_before_any_launch(lib):
    """Sizes the API accepts but whose launch grid would exceed 2^32 - 1
    work-items: every launcher refuses them (DLM_ESHAPE) before any HIP call,
    so the fake pointers are never used."""
    P = C.c_void_p
    T = 1 << 30
    for dt in (dlm.DLM_BF16, dlm.DLM_F32):
        assert lib.dlm_pregate(P(FAKE), P(FAKE), T, 64, 8, dt, P(FAKE), P(FAKE), None) == dlm.DLM_ESHAPE
        assert "2^32" in _err(lib)
        assert lib.dlm_pregate_centroid(P(FAKE), P(FAKE), T, 64, 8, 4, dt, P(FAKE), P(FAKE),
                                        None) == dlm.DLM_ESHAPE
        # x, the sets, the banks, y and the workspace at addresses far enough
        # apart that their extents at T = 2^30 rows do not overlap
        x, idx, g, A, B, y, w = FAKE, 1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44, 1 << 46
        assert lib.dlm_sgmm(P(x), P(idx), P(g), P(A), P(B), P(y), T, 8, 8, 1, 1, 1.0, dt,
                            P(w), C.c_size_t(1 << 45), None) == dlm.DLM_ESHAPE
        assert "2^32" in _err(lib)
