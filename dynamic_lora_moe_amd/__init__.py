"""MI355X (gfx950) hot path of token-level pre-gated dynamic LoRA adapters.

A thin ctypes binding of libdlm.so (declared in include/dlm.h).  It only
marshals torch tensors (device memory) and the current HIP stream into the
C ABI; every step of the path runs in the library's HIP kernels.  There is no
fallback: if the library is missing or fails to load, importing the ops raises.

  pregate(x, Wr)                  -> (idx [T][2] int32, g [T][2] fp32)
  Layers([(W, A, B), ...], E, r, scale).switch(old, new)   # in place, one launch
  sgmm(x, idx, g, A, B, y, scale)                          # y updated in place
  SgmmGroup([(x, A, B, y), ...], E, r, scale).run(idx, g)
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlm.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "dlm.h")

DLM_OK, DLM_EINVAL, DLM_ESHAPE, DLM_EDTYPE, DLM_EALIGN = 0, -1, -2, -3, -4
DLM_EWORKSPACE, DLM_EHIP, DLM_EDEVICE, DLM_ENOMEM = -5, -6, -7, -8
DLM_F32, DLM_BF16 = 0, 1
STATUS_NAMES = {0: "DLM_OK", -1: "DLM_EINVAL", -2: "DLM_ESHAPE", -3: "DLM_EDTYPE",
                -4: "DLM_EALIGN", -5: "DLM_EWORKSPACE", -6: "DLM_EHIP", -7: "DLM_EDEVICE",
                -8: "DLM_ENOMEM"}


class DLMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class dlm_proj(C.Structure):
    _fields_ = [("W", C.c_void_p), ("A", C.c_void_p), ("B", C.c_void_p),
                ("d_out", C.c_int64), ("d_in", C.c_int64)]


class dlm_sgmm_problem(C.Structure):
    _fields_ = [("x", C.c_void_p), ("A", C.c_void_p), ("B", C.c_void_p), ("y", C.c_void_p),
                ("d_in", C.c_int64), ("d_out", C.c_int64)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libdlm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with dynamic_lora_moe_amd/build.py")
    lib = C.CDLL(path)
    P, I64, I32, F = C.c_void_p, C.c_int64, C.c_int32, C.c_float
    sig = {
        "dlm_last_error": ([], C.c_char_p),
        "dlm_version": ([], C.c_char_p),
        "dlm_pregate": ([P, P, I64, I64, I32, I32, P, P, P], C.c_int),
        "dlm_pregate_centroid": ([P, P, I64, I64, I32, I32, I32, P, P, P], C.c_int),
        "dlm_layers_create": ([P, I32, I32, I32, F, I32, P], C.c_int),
        "dlm_layers_destroy": ([P], C.c_int),
        "dlm_switch": ([P, P, P, P, P, P], C.c_int),
        "dlm_switch_launches": ([P], C.c_int),
        "dlm_layers_status": ([P, P, P], C.c_int),
        "dlm_sgmm_workspace_size": ([I64, I64, I32, I32, I32, P], C.c_int),
        "dlm_sgmm": ([P, P, P, P, P, P, I64, I64, I64, I32, I32, F, I32, P, C.c_size_t, P], C.c_int),
        "dlm_sgmm_noalloc": ([P, P, P, P, P, P, I64, I64, I64, I32, I32, F, I32, P, P], C.c_int),
        "dlm_sgmm_group_create": ([P, I32, I32, I32, F, I32, P], C.c_int),
        "dlm_sgmm_group_destroy": ([P], C.c_int),
        "dlm_layers_repack": ([P, P], C.c_int),
        "dlm_layers_bind_vectors": ([P, P, P], C.c_int),
        "dlm_gemv": ([P, P], C.c_int),
        "dlm_switch_gemv": ([P, P, P, P, P, P], C.c_int),
        "dlm_switch_gemv_launches": ([P], C.c_int),
        "dlm_gemv_unmerged": ([P, P, P, P], C.c_int),
        "dlm_gemv_unmerged_launches": ([P], C.c_int),
        "dlm_sgmm_launches": ([I64, I64, I32, I32, I32], C.c_int),
        "dlm_sgmm_group_repack": ([P, P], C.c_int),
        "dlm_sgmm_group_run": ([P, P, P, I64, P, C.c_size_t, P], C.c_int),
        "dlm_sgmm_status": ([P, P, P], C.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/dlm.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dlm_\w+)\s*\(", text, flags=re.M)))


def _check(rc: int, what: str):
    if rc != DLM_OK:
        raise DLMError(rc, f"{what}: {load().dlm_last_error().decode()}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DLM_F32
    if t.dtype == torch.bfloat16:
        return DLM_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _like(t: torch.Tensor, name: str, shape, dtype, device):
    """The library takes bare pointers and cannot see a tensor's extent: every
    buffer it reads or writes is checked here against the shape it will assume."""
    _need(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _sets_out(idx, g, T: int, device, what: str):
    """Per-row expert sets: idx [T][2] int32 and g [T][2] fp32 (allocated when None)."""
    if idx is None:
        idx = torch.empty((T, 2), dtype=torch.int32, device=device)
    if g is None:
        g = torch.empty((T, 2), dtype=torch.float32, device=device)
    _like(idx, f"{what} idx", (T, 2), torch.int32, device)
    _like(g, f"{what} g", (T, 2), torch.float32, device)
    return idx, g


# ---- router -------------------------------------------------------------------

def pregate(x: torch.Tensor, Wr: torch.Tensor, idx=None, g=None, stream=None):
    """Top-2 pre-gate: x [T][d], Wr [d][E] -> idx [T][2] int32, g [T][2] fp32 (device)."""
    _need(x, "x")
    _need(Wr, "Wr")
    T, d = x.shape
    E = Wr.shape[1]
    _like(Wr, "Wr", (d, E), x.dtype, x.device)
    idx, g = _sets_out(idx, g, T, x.device, "pregate")
    _check(load().dlm_pregate(_p(x), _p(Wr), T, d, E, _dt(x), _p(idx), _p(g), _stream(stream)),
           "dlm_pregate")
    return idx, g


def pregate_centroid(x: torch.Tensor, C: torch.Tensor, idx=None, g=None, stream=None):
    """Nearest-centroid pre-gate: x [T][d], C [E][J][d] -> idx [T][2] int32 (slot 1
    empty), g [T][2] fp32 = (1, 0) (device)."""
    _need(x, "x")
    _need(C, "C")
    T, d = x.shape
    E, J, d2 = C.shape
    _like(C, "C", (E, J, d), x.dtype, x.device)
    idx, g = _sets_out(idx, g, T, x.device, "pregate_centroid")
    _check(load().dlm_pregate_centroid(_p(x), _p(C), T, d, E, J, _dt(x), _p(idx), _p(g), _stream(stream)),
           "dlm_pregate_centroid")
    return idx, g


# ---- fused switch ---------------------------------------------------------------

def _set_ptrs(s):
    if s is None:
        return None, None
    i, g = s
    _need(i, "set idx")
    _need(g, "set g")
    if i.dtype != torch.int32 or g.dtype != torch.float32 or i.numel() < 2 or g.numel() < 2:
        raise ValueError("a set is (int32 idx[2], fp32 g[2]) on the device")
    return _p(i), _p(g)


class Layers:
    """Every adapted weight of every layer, switched together by one launch."""

    def __init__(self, projs, E: int, r: int, scale: float):
        self._keep = list(projs)
        arr = (dlm_proj * len(self._keep))()
        dt = None
        for k, (W, A, B) in enumerate(self._keep):
            _need(W, f"weight {k} W")
            if W.dim() != 2:
                raise ValueError(f"weight {k}: W must be [d_out][d_in]")
            d_out, d_in = W.shape
            W0 = self._keep[0][0]
            _like(W, f"weight {k} W", (d_out, d_in), W0.dtype, W0.device)
            _like(A, f"weight {k} A", (E, r, d_in), W.dtype, W.device)
            _like(B, f"weight {k} B", (E, d_out, r), W.dtype, W.device)
            dt = _dt(W) if dt is None else dt
            arr[k] = dlm_proj(W.data_ptr(), A.data_ptr(), B.data_ptr(), W.shape[0], W.shape[1])
        h = C.c_void_p()
        _check(load().dlm_layers_create(arr, len(self._keep), E, r, float(scale), dt, C.byref(h)),
               "dlm_layers_create")
        self._h = h
        self.E, self.r, self.scale = E, r, scale

    def switch(self, old=None, new=None, stream=None):
        """old/new: (idx int32[2], g fp32[2]) device tensors, or None for the empty set."""
        oi, og = _set_ptrs(old)
        ni, ng = _set_ptrs(new)
        _check(load().dlm_switch(self._h, oi, og, ni, ng, _stream(stream)), "dlm_switch")

    def status(self, stream=None) -> int:
        code = C.c_int32(0)
        _check(load().dlm_layers_status(self._h, C.byref(code), _stream(stream)), "dlm_layers_status")
        return code.value

    def launches_per_switch(self) -> int:
        return load().dlm_switch_launches(self._h)

    def bind_vectors(self, xs, ys):
        """Bind an input x_i [d_in] (the weights' dtype) and an output y_i [d_out]
        (fp32) device tensor to every weight, for gemv() and switch_gemv()."""
        if not len(xs) == len(ys) == len(self._keep):
            raise ValueError("one x and one y per weight")
        for k, ((W, _, _), x, y) in enumerate(zip(self._keep, xs, ys)):
            _like(x, f"x {k}", (W.shape[1],), W.dtype, W.device)
            _like(y, f"y {k}", (W.shape[0],), torch.float32, W.device)
        xa = (C.c_void_p * len(xs))(*[x.data_ptr() for x in xs])
        ya = (C.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
        _check(load().dlm_layers_bind_vectors(self._h, xa, ya), "dlm_layers_bind_vectors")
        self._vecs = (list(xs), list(ys))

    def gemv(self, stream=None):
        """y_i = W_i x_i for every weight (bound vectors)."""
        _check(load().dlm_gemv(self._h, _stream(stream)), "dlm_gemv")

    def switch_gemv(self, old=None, new=None, stream=None):
        """switch(old, new), then y_i = W'_i x_i (bound vectors)."""
        oi, og = _set_ptrs(old)
        ni, ng = _set_ptrs(new)
        _check(load().dlm_switch_gemv(self._h, oi, og, ni, ng, _stream(stream)), "dlm_switch_gemv")

    def launches_per_switch_gemv(self) -> int:
        return load().dlm_switch_gemv_launches(self._h)

    def gemv_unmerged(self, new, stream=None):
        """y_i = W_i x_i + s sum_k g_k B_k (A_k x_i) for the set new = (idx
        int32[2], g fp32[2]) on the device (bound vectors); W is not modified."""
        ni, ng = _set_ptrs(new)
        if not ni:
            raise ValueError("gemv_unmerged needs a set (idx, g)")
        _check(load().dlm_gemv_unmerged(self._h, ni, ng, _stream(stream)), "dlm_gemv_unmerged")

    def launches_per_gemv_unmerged(self) -> int:
        return load().dlm_gemv_unmerged_launches(self._h)

    def repack(self, stream=None):
        """Refresh the packed A copy (ranks 17..64, bf16) after changing an A bank in place."""
        _check(load().dlm_layers_repack(self._h, _stream(stream)), "dlm_layers_repack")

    def close(self):
        if getattr(self, "_h", None):
            _check(load().dlm_layers_destroy(self._h), "dlm_layers_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


# ---- SGMM ------------------------------------------------------------------------

def sgmm_workspace_size(T: int, d_in_max: int, E: int, r: int, n_problems: int = 1) -> int:
    b = C.c_size_t(0)
    _check(load().dlm_sgmm_workspace_size(T, d_in_max, E, r, n_problems, C.byref(b)),
           "dlm_sgmm_workspace_size")
    return b.value


def sgmm_workspace(T: int, d_in_max: int, E: int, r: int, n_problems: int = 1,
                   device="cuda") -> torch.Tensor:
    n = sgmm_workspace_size(T, d_in_max, E, r, n_problems)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _ws_bytes(workspace) -> int:
    _need(workspace, "workspace")
    return workspace.numel() * workspace.element_size()


def sgmm(x, idx, g, A, B, y, scale: float, workspace=None, stream=None):
    """y += sum_k s g_k (x A_k^T) B_k^T row by row, in place (returns y).

    With a workspace the call only enqueues; read the device's decision on the
    sets with sgmm_status(workspace).  Without one it allocates a workspace,
    waits for the launches (so the temporary outlives them) and raises
    DLMError(DLM_EDEVICE) if the device rejected a set (y is then unchanged)."""
    _need(x, "x")
    _need(A, "A")
    _need(B, "B")
    T, d_in = x.shape
    E, r, _ = A.shape
    d_out = B.shape[1]
    _like(A, "A", (E, r, d_in), x.dtype, x.device)
    _like(B, "B", (E, d_out, r), x.dtype, x.device)
    _like(y, "y", (T, d_out), x.dtype, x.device)
    _like(idx, "idx", (T, 2), torch.int32, x.device)
    _like(g, "g", (T, 2), torch.float32, x.device)
    own = workspace is None
    if own:
        workspace = sgmm_workspace(T, d_in, E, r, 1, x.device)
    _check(load().dlm_sgmm(_p(x), _p(idx), _p(g), _p(A), _p(B), _p(y), T, d_in, d_out, E, r,
                           float(scale), _dt(x), _p(workspace), _ws_bytes(workspace), _stream(stream)),
           "dlm_sgmm")
    if own and T > 0 and sgmm_status(workspace, stream) != DLM_OK:
        raise DLMError(DLM_EDEVICE, "dlm_sgmm: the device rejected an expert set (index outside [-1, E) or "
                                    "a non-finite gate); y is unchanged")
    return y


def sgmm_noalloc(x, idx, g, A, B, y, scale: float, status=None, stream=None):
    """sgmm() with the workspace in the library's own scratch array (no device
    allocation by the call; calls overlapping on one device race).  status: an
    optional int32 [1] device tensor receiving 0, or nonzero if a set was rejected."""
    _need(x, "x")
    _need(A, "A")
    _need(B, "B")
    T, d_in = x.shape
    E, r, _ = A.shape
    d_out = B.shape[1]
    _like(A, "A", (E, r, d_in), x.dtype, x.device)
    _like(B, "B", (E, d_out, r), x.dtype, x.device)
    _like(y, "y", (T, d_out), x.dtype, x.device)
    _like(idx, "idx", (T, 2), torch.int32, x.device)
    _like(g, "g", (T, 2), torch.float32, x.device)
    if status is not None:
        _like(status, "status", (1,), torch.int32, x.device)
    _check(load().dlm_sgmm_noalloc(_p(x), _p(idx), _p(g), _p(A), _p(B), _p(y), T, d_in, d_out, E, r,
                                   float(scale), _dt(x), _p(status), _stream(stream)), "dlm_sgmm_noalloc")
    return y


def sgmm_launches(T: int, d_in_max: int, r: int, n_problems: int = 1, dtype=torch.bfloat16) -> int:
    """Kernel launches of one sgmm / sgmm_noalloc (n_problems = 1) or
    SgmmGroup.run call at rank r."""
    dt = {torch.float32: DLM_F32, torch.bfloat16: DLM_BF16}.get(dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {dtype}")
    n = load().dlm_sgmm_launches(T, d_in_max, r, n_problems, dt)
    if n < 0:
        raise DLMError(DLM_EINVAL, load().dlm_last_error().decode())
    return n


def sgmm_status(workspace, stream=None) -> int:
    code = C.c_int32(0)
    _check(load().dlm_sgmm_status(_p(workspace), C.byref(code), _stream(stream)), "dlm_sgmm_status")
    return code.value


class SgmmGroup:
    """Many (x, A, B, y) problems run on the same rows' expert sets (decide once)."""

    def __init__(self, problems, E: int, r: int, scale: float):
        self._keep = list(problems)
        arr = (dlm_sgmm_problem * len(self._keep))()
        dt = None
        x0 = self._keep[0][0]
        _need(x0, "problem 0 x")
        for k, (x, A, B, y) in enumerate(self._keep):
            _need(x, f"problem {k} x")
            _need(B, f"problem {k} B")
            if x.dim() != 2 or B.dim() != 3:
                raise ValueError(f"problem {k}: x must be [T][d_in] and B [E][d_out][r]")
            T_k, d_in = x.shape
            d_out = B.shape[1]
            _like(x, f"problem {k} x", (T_k, d_in), x0.dtype, x0.device)
            _like(A, f"problem {k} A", (E, r, d_in), x.dtype, x.device)
            _like(B, f"problem {k} B", (E, d_out, r), x.dtype, x.device)
            _like(y, f"problem {k} y", (T_k, d_out), x.dtype, x.device)
            dt = _dt(x) if dt is None else dt
            arr[k] = dlm_sgmm_problem(x.data_ptr(), A.data_ptr(), B.data_ptr(), y.data_ptr(),
                                      x.shape[1], y.shape[1])
        h = C.c_void_p()
        _check(load().dlm_sgmm_group_create(arr, len(self._keep), E, r, float(scale), dt, C.byref(h)),
               "dlm_sgmm_group_create")
        self._h = h
        self.E, self.r, self.n = E, r, len(self._keep)
        self.d_in_max = max(x.shape[1] for x, _, _, _ in self._keep)
        self.rows = min(x.shape[0] for x, _, _, _ in self._keep)  # rows every problem holds
        self.device = x0.device

    def workspace(self, T: int, device="cuda"):
        return sgmm_workspace(T, self.d_in_max, self.E, self.r, self.n, device)

    def repack(self, stream=None):
        """Refresh the packed A copies after the A banks were changed in place."""
        _check(load().dlm_sgmm_group_repack(self._h, _stream(stream)), "dlm_sgmm_group_repack")

    def run(self, idx, g, T: int | None = None, workspace=None, stream=None):
        """Run every problem on rows [0, T) of (idx, g); returns the workspace,
        whose status word sgmm_status() reads (a rejected set leaves every y
        unchanged)."""
        _need(idx, "idx")
        T = idx.shape[0] if T is None else T
        if not 0 <= T <= self.rows:
            raise ValueError(f"T={T} rows, but the group's problems hold {self.rows}")
        _like(idx[:T], "idx", (T, 2), torch.int32, self.device)
        _like(g[:T], "g", (T, 2), torch.float32, self.device)
        own = workspace is None
        if own:
            workspace = self.workspace(T, idx.device)
        _check(load().dlm_sgmm_group_run(self._h, _p(idx), _p(g), T, _p(workspace),
                                         _ws_bytes(workspace), _stream(stream)), "dlm_sgmm_group_run")
        if own and stream is not None and stream != torch.cuda.current_stream():
            # a workspace made here on the current stream is used on `stream`:
            # keep the allocator from handing it out again before those launches end
            workspace.record_stream(stream)
        return workspace

    def close(self):
        if getattr(self, "_h", None):
            _check(load().dlm_sgmm_group_destroy(self._h), "dlm_sgmm_group_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass
