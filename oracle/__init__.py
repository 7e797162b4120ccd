"""Python access to the binary64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg.  The product path (the HIP library and its
binding) never imports it.

Arrays are CPU torch tensors or numpy arrays; bf16 tensors are passed as their
16-bit patterns.  Every function returns fresh outputs and leaves inputs alone
unless it says "in place".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT_F32, DT_BF16 = 0, 1


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with gcc (binary64, OpenMP over rows)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None):
    """Load the oracle library, building it first if it is missing or stale."""
    global _lib
    if path is not None:
        return _bind(C.CDLL(path))
    if _lib is None:
        if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(C.CDLL(_LIB))
    return _lib


def _bind(lib):
    P, I64, I32, D = C.c_void_p, C.c_int64, C.c_int32, C.c_double
    lib.dlmref_pregate.argtypes = [P, P, I64, I64, I32, I32, P, P, P, P, P]
    lib.dlmref_switch_rows.argtypes = [P, P, I64, P, P, I64, I64, I32, I32, D, I32,
                                       P, P, P, P, P, P]
    lib.dlmref_sgmm_rows.argtypes = [P, P, P, P, P, P, I64, I64, I64, I32, I32, D, I32, P, P]
    lib.dlmref_pregate_centroid.argtypes = [P, P, I64, I64, I32, I32, I32, P, P, P, P]
    lib.dlmref_pregate_centroid.restype = C.c_int
    lib.dlmref_gemv.argtypes = [P, P, I64, I64, I32, P, P, P]
    lib.dlmref_gemv.restype = C.c_int
    lib.dlmref_round.argtypes = [P, I64, I32, P]
    lib.dlmref_threads.restype = C.c_int
    lib.dlmref_set_threads.argtypes = [C.c_int]
    for f in (lib.dlmref_pregate, lib.dlmref_switch_rows, lib.dlmref_sgmm_rows):
        f.restype = C.c_int
    return lib


# ---- marshalling ----------------------------------------------------------

def _np(t):
    """Contiguous numpy view with bf16 as uint16 bit patterns; returns (array, dtype code)."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), DT_BF16
        if t.dtype == torch.float32:
            return t.numpy(), DT_F32
        return t.numpy(), None
    a = np.ascontiguousarray(t)
    if a.dtype == np.float32:
        return a, DT_F32
    if a.dtype == np.uint16:
        return a, DT_BF16
    return a, None


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _to_torch(a: np.ndarray, dt: int) -> torch.Tensor:
    if dt == DT_BF16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())


def _set(s):
    """(idx, g) pair of length-2 sequences or None -> (int32 array, fp32 array) or (None, None)."""
    if s is None:
        return None, None
    i, g = s
    i = np.ascontiguousarray(np.asarray(i, dtype=np.int32).reshape(2))
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float32).reshape(2))
    return i, g


# ---- API -------------------------------------------------------------------

def pregate(x, Wr, with_stats: bool = False, lib=None):
    """Router: x [T][d], Wr [d][E] -> idx [T][2] int32, g [T][2] fp32 (torch).

    with_stats also returns (logits [T][E] f64, margin [T], bound [T])."""
    lib = lib or load()
    xa, dt = _np(x)
    wa, dt2 = _np(Wr)
    assert dt is not None and dt == dt2
    T, d = xa.shape
    E = wa.shape[1]
    idx = np.empty((T, 2), np.int32)
    g = np.empty((T, 2), np.float32)
    lg = np.empty((T, E), np.float64) if with_stats else None
    mg = np.empty((T,), np.float64) if with_stats else None
    bd = np.empty((T,), np.float64) if with_stats else None
    rc = lib.dlmref_pregate(_ptr(xa), _ptr(wa), T, d, E, dt, _ptr(idx), _ptr(g),
                            _ptr(lg), _ptr(mg), _ptr(bd))
    if rc != 0:
        raise ValueError(f"dlmref_pregate failed ({rc})")
    out = (torch.from_numpy(idx), torch.from_numpy(g))
    if with_stats:
        return out + (torch.from_numpy(lg), torch.from_numpy(mg), torch.from_numpy(bd))
    return out


def pregate_centroid(x, C, with_stats: bool = False, lib=None):
    """Nearest-centroid router: x [T][d], C [E][J][d] -> idx [T][2] int32 (slot 1
    empty), g [T][2] fp32 = (1, 0).  with_stats also returns (dist [T][E] f64,
    margin [T] f64)."""
    lib = lib or load()
    xa, dt = _np(x)
    ca, dtc = _np(C)
    assert dt is not None and dt == dtc
    T, d = xa.shape
    E, J, d2 = ca.shape
    assert d2 == d
    idx = np.empty((T, 2), np.int32)
    g = np.empty((T, 2), np.float32)
    ds = np.empty((T, E), np.float64) if with_stats else None
    mg = np.empty((T,), np.float64) if with_stats else None
    rc = lib.dlmref_pregate_centroid(_ptr(xa), _ptr(ca), T, d, E, J, dt, _ptr(idx), _ptr(g), _ptr(ds), _ptr(mg))
    if rc != 0:
        raise ValueError(f"dlmref_pregate_centroid failed ({rc})")
    out = (torch.from_numpy(idx), torch.from_numpy(g))
    if with_stats:
        return out + (torch.from_numpy(ds), torch.from_numpy(mg))
    return out


def switch_rows(W_rows, rows, A, B, d_out, scale, old, new, with_stats=False, lib=None):
    """Switch the given rows of one adapted weight.

    W_rows [n][d_in] is the pre-state of rows `rows` (not modified); A [E][r][d_in],
    B [E][d_out][r]; old/new are (idx[2], g[2]) or None.  Returns the switched rows
    (same dtype), and with_stats also (exact f64 [n][d_in], absum f64 [n][d_in])."""
    lib = lib or load()
    wa, dt = _np(W_rows)
    wa = wa.copy()
    aa, dta = _np(A)
    ba, dtb = _np(B)
    assert dt == dta == dtb and dt is not None
    E, r, d_in = aa.shape
    assert ba.shape == (E, d_out, r) and wa.shape[1] == d_in
    rws = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rws.shape[0]
    oi, og = _set(old)
    ni, ng = _set(new)
    ex = np.empty((n, d_in), np.float64) if with_stats else None
    ab = np.empty((n, d_in), np.float64) if with_stats else None
    rc = lib.dlmref_switch_rows(_ptr(wa), _ptr(rws), n, _ptr(aa), _ptr(ba), d_out, d_in, E, r,
                                float(scale), dt, _ptr(oi), _ptr(og), _ptr(ni), _ptr(ng),
                                _ptr(ex), _ptr(ab))
    if rc != 0:
        raise ValueError(f"dlmref_switch_rows failed ({rc})")
    out = _to_torch(wa, dt)
    if with_stats:
        return out, torch.from_numpy(ex), torch.from_numpy(ab)
    return out


def switch(W, A, B, scale, old, new, with_stats=False, lib=None):
    """Switch every row of W [d_out][d_in]."""
    d_out = W.shape[0]
    return switch_rows(W, np.arange(d_out), A, B, d_out, scale, old, new, with_stats, lib)


def sgmm(x, idx, g, A, B, y, scale, with_stats=False, lib=None):
    """y_out = round(y + sum_k s g_k (x A_k^T) B_k^T) row by row (y not modified)."""
    lib = lib or load()
    xa, dt = _np(x)
    aa, dta = _np(A)
    ba, dtb = _np(B)
    ya, dty = _np(y)
    assert dt == dta == dtb == dty and dt is not None
    ya = ya.copy()
    n, d_in = xa.shape
    E, r, d_in2 = aa.shape
    d_out = ba.shape[1]
    assert d_in2 == d_in and ba.shape == (E, d_out, r) and ya.shape == (n, d_out)
    ia = np.ascontiguousarray(np.asarray(idx, dtype=np.int32).reshape(n, 2))
    ga = np.ascontiguousarray(np.asarray(g, dtype=np.float32).reshape(n, 2))
    ex = np.empty((n, d_out), np.float64) if with_stats else None
    ab = np.empty((n, d_out), np.float64) if with_stats else None
    rc = lib.dlmref_sgmm_rows(_ptr(xa), _ptr(ia), _ptr(ga), _ptr(aa), _ptr(ba), _ptr(ya),
                              n, d_in, d_out, E, r, float(scale), dt, _ptr(ex), _ptr(ab))
    if rc != 0:
        raise ValueError(f"dlmref_sgmm_rows failed ({rc})")
    out = _to_torch(ya, dt)
    if with_stats:
        return out, torch.from_numpy(ex), torch.from_numpy(ab)
    return out


def gemv(W, x, with_stats=False, lib=None):
    """y = round_fp32(W @ x) for W [d_out][d_in], x [d_in] (fp32 torch out);
    with_stats also returns (exact f64 [d_out], absum f64 [d_out])."""
    lib = lib or load()
    wa, dt = _np(W)
    xa, dtx = _np(x)
    assert dt == dtx and dt is not None
    d_out, d_in = wa.shape
    assert xa.shape == (d_in,)
    y = np.empty((d_out,), np.float32)
    ex = np.empty((d_out,), np.float64) if with_stats else None
    ab = np.empty((d_out,), np.float64) if with_stats else None
    rc = lib.dlmref_gemv(_ptr(wa), _ptr(xa), d_out, d_in, dt, _ptr(y), _ptr(ex), _ptr(ab))
    if rc != 0:
        raise ValueError(f"dlmref_gemv failed ({rc})")
    out = torch.from_numpy(y)
    if with_stats:
        return out, torch.from_numpy(ex), torch.from_numpy(ab)
    return out


def round_to(v: np.ndarray, dt: int, lib=None):
    """Round binary64 values once to fp32 (dt=0) or bf16 (dt=1, returned as uint16 bits)."""
    lib = lib or load()
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.empty(v.shape, np.float32 if dt == DT_F32 else np.uint16)
    lib.dlmref_round(_ptr(v), v.size, dt, _ptr(out))
    return out


def threads(lib=None) -> int:
    return (lib or load()).dlmref_threads()


def set_threads(n: int, lib=None):
    (lib or load()).dlmref_set_threads(int(n))
