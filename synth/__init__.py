"""Seeded synthetic inputs for the pre-gated dynamic-LoRA hot path.

This module only draws random inputs: weights, adapter banks, router weights,
token activations and the per-row expert sets of the batched workloads.  It
holds none of the method's arithmetic (no routing, no merging, no adapter
products); both the HIP path and the CPU oracle receive what it produces.

Every stream is counter-based: numpy's Philox4x32 on the host and torch's
Philox on the device, keyed by (base seed, workload id, tensor kind, layer,
projection, ...).  Host and device streams are different streams; a value is
never regenerated on the other side, the consumer copies what it needs.

Distributions (the pages give none; these are the workload definitions):
  backbone W, adapter A/B, router Wr : N(0, 0.02)
  token activations x               : N(0, 1)
  SGMM incoming y (stand-in for the base projection output x.W^T) :
                                      N(0, 0.02^2 * d_in)
Values are drawn in fp32 (torch) or fp64 (numpy) and rounded to the storage
dtype with round-to-nearest-even.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 20260312

_KINDS = {"W": 1, "A": 2, "B": 3, "Wr": 4, "x": 5, "y0": 6, "z": 7, "sets": 8,
          "misc": 9}


def substream_seed(*keys) -> int:
    """64-bit seed for a substream named by a tuple of ints/strings."""
    h = hashlib.sha256(repr((SEED_BASE,) + tuple(keys)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def host_rng(*keys) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=substream_seed(*keys)))


def normal_host(shape, std, dtype: torch.dtype, *keys) -> torch.Tensor:
    """N(0, std^2) drawn in fp64 on the host, rounded once to `dtype` (CPU tensor)."""
    a = host_rng(*keys).standard_normal(size=shape) * std
    t64 = torch.from_numpy(a)
    if dtype == torch.float64:
        return t64
    if dtype == torch.float32:
        return t64.to(torch.float32)
    # fp64 -> bf16 through fp32 would round twice; go through fp64 -> bf16
    # directly (torch rounds to nearest even from the source precision).
    return t64.to(dtype)


def normal_device(shape, std, dtype: torch.dtype, device, *keys,
                  chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(0, std^2) drawn on the device in fp32 (torch Philox), rounded to `dtype`.

    Large tensors are filled in chunks so the fp32 staging stays bounded."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    gen = torch.Generator(device=device)
    gen.manual_seed(substream_seed(*keys))
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        tmp = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        flat[s:e].copy_(tmp)
        del tmp
    return out


def fill_normal_device_(t: torch.Tensor, std, *keys, chunk_elems: int = 1 << 28):
    """Refill an existing device tensor in place with the same stream as normal_device."""
    flat = t.view(-1)
    n = flat.numel()
    gen = torch.Generator(device=t.device)
    gen.manual_seed(substream_seed(*keys))
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        tmp = torch.randn(e - s, generator=gen, device=t.device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        flat[s:e].copy_(tmp)
        del tmp
    return t


# --------------------------------------------------------------------------
# Expert-set recipes for the batched (unmerged) workloads.
# --------------------------------------------------------------------------

def _two_logit_weights(rng: np.random.Generator, n: int):
    """Per-row weights as the softmax of two N(0,1) logits, larger first.

    Returned as fp32; ties keep the drawing order."""
    z = rng.standard_normal(size=(n, 2))
    zmax = z.max(axis=1, keepdims=True)
    ez = np.exp(z - zmax)
    w = ez / ez.sum(axis=1, keepdims=True)
    return w


def _order_by_weight(e: np.ndarray, w: np.ndarray):
    """Slot 0 gets the larger weight; equal weights -> lower expert index first."""
    swap = (w[:, 1] > w[:, 0]) | ((w[:, 1] == w[:, 0]) & (e[:, 1] < e[:, 0]))
    e2 = e.copy()
    w2 = w.copy()
    e2[swap, 0], e2[swap, 1] = e[swap, 1], e[swap, 0]
    w2[swap, 0], w2[swap, 1] = w[swap, 1], w[swap, 0]
    return e2, w2


def zipf_pair_sets(T: int, E: int, s: float, *keys):
    """Prefill recipe: each row draws two distinct experts from Zipf(s) over ranks
    1..E (rank k <-> expert k-1; the second draw is without replacement) and
    weights softmax(N(0,1)^2), slot 0 the larger.  Returns (idx int32 [T][2],
    g fp32 [T][2]) as CPU tensors."""
    rng = host_rng(*keys, "zipf")
    p = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    p = p / p.sum()
    e0 = rng.choice(E, size=T, p=p)
    e1 = np.empty(T, dtype=np.int64)
    for t in range(T):
        q = p.copy()
        q[e0[t]] = 0.0
        e1[t] = rng.choice(E, p=q / q.sum())
    w = _two_logit_weights(rng, T)
    e, w = _order_by_weight(np.stack([e0, e1], 1), w)
    return (torch.from_numpy(e.astype(np.int32)),
            torch.from_numpy(w.astype(np.float32)))


def markov_pair_sets(steps: int, rows: int, E: int, p_keep: float, *keys):
    """Mixed-decode recipe: each row starts on a uniform unordered pair of distinct
    experts; each step it keeps its pair with probability p_keep, else moves to one
    of the other pairs uniformly.  Weights are redrawn every step as softmax of two
    N(0,1) logits.  Returns idx int32 [steps][rows][2], g fp32 [steps][rows][2]."""
    rng = host_rng(*keys, "markov")
    pairs = [(a, b) for a in range(E) for b in range(a + 1, E)]
    P = len(pairs)
    cur = rng.integers(0, P, size=rows)
    idx = np.empty((steps, rows, 2), dtype=np.int32)
    g = np.empty((steps, rows, 2), dtype=np.float32)
    for st in range(steps):
        if st > 0:
            move = rng.random(size=rows) >= p_keep
            jump = rng.integers(0, P - 1, size=rows)
            jump = jump + (jump >= cur)  # uniform over the other P-1 pairs
            cur = np.where(move, jump, cur)
        e = np.array([pairs[c] for c in cur], dtype=np.int64)
        # which member of the pair is slot 0 is decided by the drawn weights
        flip = rng.random(size=rows) < 0.5
        e[flip] = e[flip][:, ::-1]
        w = _two_logit_weights(rng, rows)
        e, w = _order_by_weight(e, w)
        idx[st] = e
        g[st] = w
    return torch.from_numpy(idx), torch.from_numpy(g)


# --------------------------------------------------------------------------
# Workload definitions
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    cfg_id: int
    dtype: torch.dtype
    layers: int
    projs: list            # [(name, d_out, d_in)]
    E: int
    r: int
    scale: float
    d_model: int
    T: int                 # tokens (decode chain length, or prefill rows, or batch rows)
    steps: int = 1         # decode steps for the batched-decode workload
    extra: dict = field(default_factory=dict)

    @property
    def n_mats(self):
        return self.layers * len(self.projs)

    def switch_w_elems(self):
        return self.layers * sum(o * i for _, o, i in self.projs)


_P7B = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
        ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
_P70B = [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
         ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]

WORKLOADS = {
    # tiny fp32: 2 layers x one 64x64 projection, E=4, r=4, router 64x4 on 16 tokens
    "tiny-fp32": Workload("tiny-fp32", 0, torch.float32, 2, [("p", 64, 64)], 4, 4, 1.0, 64, 16),
    # 7B-shaped decode, batch 1: 32 layers x 7 projections, E=8, r=16, scale 2, 256 tokens
    "7b-decode": Workload("7b-decode", 1, torch.bfloat16, 32, _P7B, 8, 16, 2.0, 4096, 256),
    # prefill SGMM: one layer x 7 projections, 4096 tokens, E=8, r=16, Zipf(1.1) pairs
    "sgmm-prefill": Workload("sgmm-prefill", 2, torch.bfloat16, 1, _P7B, 8, 16, 1.0, 4096, 4096,
                             extra={"zipf_s": 1.1}),
    # 70B-shaped decode, batch 1: 80 layers x 7 projections, E=16, r=64, 128 tokens
    "70b-decode": Workload("70b-decode", 3, torch.bfloat16, 80, _P70B, 16, 64, 1.0, 8192, 128),
    # mixed decode batch 64: 32 layers x 7 projections, E=8, r=16, 128 steps, keep p=0.9
    "mixed-decode": Workload("mixed-decode", 4, torch.bfloat16, 32, _P7B, 8, 16, 1.0, 4096, 64,
                             steps=128, extra={"p_keep": 0.9}),
}


# --------------------------------------------------------------------------
# Device-resident inputs of a workload
# --------------------------------------------------------------------------

def switch_model(wl: Workload, device="cuda", layers=None):
    """[(layer, proj_name, W, A, B)] for every adapted weight of the decode workloads:
    W [d_out][d_in] ~ N(0, .02), A [E][r][d_in], B [E][d_out][r] ~ N(0, .02)."""
    out = []
    for l in (range(wl.layers) if layers is None else layers):
        for pi, (name, o, i) in enumerate(wl.projs):
            W = normal_device((o, i), 0.02, wl.dtype, device, wl.cfg_id, "W", l, pi)
            A = normal_device((wl.E, wl.r, i), 0.02, wl.dtype, device, wl.cfg_id, "A", l, pi)
            B = normal_device((wl.E, o, wl.r), 0.02, wl.dtype, device, wl.cfg_id, "B", l, pi)
            out.append((l, name, W, A, B))
    return out


def refill_switch_weights_(wl: Workload, model):
    """Regenerate every W of `model` in place (same streams as switch_model)."""
    for l, name, W, _, _ in model:
        pi = [p[0] for p in wl.projs].index(name)
        fill_normal_device_(W, 0.02, wl.cfg_id, "W", l, pi)


def router_inputs(wl: Workload, device="cuda"):
    """x [T][d] ~ N(0, 1) and Wr [d][E] ~ N(0, .02) of the decode workloads."""
    x = normal_device((wl.T, wl.d_model), 1.0, wl.dtype, device, wl.cfg_id, "x")
    Wr = normal_device((wl.d_model, wl.E), 0.02, wl.dtype, device, wl.cfg_id, "Wr")
    return x, Wr


def sgmm_problems(wl: Workload, device="cuda", layers=None):
    """[(layer, proj_name, x, A, B, y0)] of the batched workloads: x [T][d_in] ~ N(0, 1),
    y0 [T][d_out] ~ N(0, .02^2 d_in) standing in for the base output, A/B ~ N(0, .02).
    For the decode workloads (one router set per token) the same recipe gives the
    unmerged form of their layers, T = the workload's token count."""
    out = []
    for l in (range(wl.layers) if layers is None else layers):
        for pi, (name, o, i) in enumerate(wl.projs):
            x = normal_device((wl.T, i), 1.0, wl.dtype, device, wl.cfg_id, "x", l, pi)
            A = normal_device((wl.E, wl.r, i), 0.02, wl.dtype, device, wl.cfg_id, "A", l, pi)
            B = normal_device((wl.E, o, wl.r), 0.02, wl.dtype, device, wl.cfg_id, "B", l, pi)
            y = normal_device((wl.T, o), 0.02 * i ** 0.5, wl.dtype, device, wl.cfg_id, "y0", l, pi)
            out.append((l, name, x, A, B, y))
    return out


def batched_sets(wl: Workload):
    """Expert sets of the batched workloads as CPU tensors:
    prefill -> idx [T][2], g [T][2]; mixed decode -> idx [steps][T][2], g [steps][T][2]."""
    if wl.name == "sgmm-prefill":
        return zipf_pair_sets(wl.T, wl.E, wl.extra["zipf_s"], wl.cfg_id, "sets")
    if wl.name == "mixed-decode":
        return markov_pair_sets(wl.steps, wl.T, wl.E, wl.extra["p_keep"], wl.cfg_id, "sets")
    raise ValueError(wl.name)
