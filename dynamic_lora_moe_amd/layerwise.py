"""Layer-wise dynamic adapters: the per-layer routing form that token-level
pre-gating replaces, built from this library's kernels only.

AdaFuse (problem statement and experiments sections) attributes the decode
slowdown of earlier dynamic-adapter systems to this form: every layer makes its
own routing decision and applies its adapters unmerged, so a token costs many
small sequential kernel launches.  Per token and per layer l:

  1. router: dlm_pregate on the layer's router input with the layer's own
     router weights Wr_l (T = 1) -> the layer's top-2 set (idx_l, g_l);
  2. base product: dlm_gemv, y_base = W x for every adapted projection of the
     layer, on the unchanged base weights (fp32 outputs);
  3. unmerged adapters: y_lora += s g_k (x A_k^T) B_k^T for the layer's set,
     either one dlm_sgmm call per projection (T = 1; the per-module form) or one
     grouped SGMM per layer (``grouped=True``: one segmentation for the
     layer's projections).

With ``fused=True`` steps 2 and 3 are one dlm_gemv_unmerged call per layer:
the adapters' down-projections of the layer's inputs, then the base product
with the adapters' up-projections added in the same pass (two launches for the
layer, the result in the fp32 base outputs; the weights stay unmerged).

With ``route_once=True`` the router runs once per token (the first layer's
router weights) and every layer applies that set: the pre-gated decision of
AdaFuse (Chinese digest, method section; Korean digest section 2-ga) with the
adapters still unmerged, so one router launch per token instead of one per layer.

Unfused, the layer's adapted output is y_base + y_lora; the two stay in
separate buffers (the adding is one more element-wise pass, not timed here).  Nothing
here computes: each step is an entry point of libdlm.so, and the class only
holds buffers and issues the calls in order on one stream.
"""
from __future__ import annotations

import torch

from . import DLM_OK, Layers, SgmmGroup, pregate, sgmm, sgmm_launches, sgmm_status, sgmm_workspace


class LayerwiseDecode:
    """One decode token through every layer with per-layer routing (or, with
    route_once, one routing decision for all layers).

    layers:  per layer, the adapted projections [(W, A, B)] (W [d_out][d_in],
             A [E][r][d_in], B [E][d_out][r], one dtype); W is never modified.
    routers: per layer, Wr_l [d_router][E] (the weights' dtype).
    xs:      per layer, one input vector [d_in] per projection (the weights'
             dtype), read in place by the base product and the adapters.
    """

    def __init__(self, layers, routers, xs, E: int, r: int, scale: float, grouped: bool = False,
                 route_once: bool = False, fused: bool = False):
        if not len(layers) == len(routers) == len(xs):
            raise ValueError("one projection list, one router and one input list per layer")
        if fused and grouped:
            raise ValueError("fused applies the adapters inside the product; grouped has no meaning there")
        self.E, self.r, self.scale, self.grouped, self.fused = E, r, float(scale), grouped, fused
        self.route_once = route_once
        self.routers = list(routers)
        self.xs = [list(x) for x in xs]
        W0 = layers[0][0][0]
        dev, dt = W0.device, W0.dtype
        self.base, self.y_base, self.y_lora, self.groups = [], [], [], []
        self.idx = [torch.zeros((1, 2), dtype=torch.int32, device=dev) for _ in layers]
        self.g = [torch.zeros((1, 2), dtype=torch.float32, device=dev) for _ in layers]
        self.projs = [list(p) for p in layers]
        d_in_max = 0
        for projs, xl in zip(self.projs, self.xs):
            if len(xl) != len(projs):
                raise ValueError("one input vector per projection")
            h = Layers(projs, E, r, scale)
            yb = [torch.zeros(W.shape[0], dtype=torch.float32, device=dev) for W, _, _ in projs]
            h.bind_vectors(xl, yb)
            yl = [] if fused else [torch.zeros((1, W.shape[0]), dtype=dt, device=dev) for W, _, _ in projs]
            self.base.append(h)
            self.y_base.append(yb)
            self.y_lora.append(yl)
            if grouped:
                self.groups.append(SgmmGroup([(x[None], A, B, y) for (W, A, B), x, y in zip(projs, xl, yl)],
                                             E, r, scale))
            d_in_max = max(d_in_max, max(W.shape[1] for W, _, _ in projs))
        self.d_in_max, self.dtype = d_in_max, dt
        n_ws = max(len(p) for p in self.projs) if grouped else 1
        self.ws = None if fused else sgmm_workspace(1, d_in_max, E, r, n_ws, dev)

    def step(self, router_x, stream=None, side=None):
        """Enqueue one token: router_x [1][d_router] is every layer's router input.

        side: a second stream (default priority) for the adapters.  A layer's
        base product and its adapters read only the layer's input, so with
        side the adapters run beside the base product: side waits for the
        router, and the next layer waits for both (the adapters' output feeds
        the next layer's input in a model)."""
        main = stream if stream is not None else torch.cuda.current_stream()
        ad = side if side is not None else main
        if side is not None and not hasattr(self, "_ev"):
            self._ev = [(torch.cuda.Event(), torch.cuda.Event()) for _ in self.projs]
        for l, projs in enumerate(self.projs):
            s = 0 if self.route_once else l  # the set this layer applies
            if l == s:
                pregate(router_x, self.routers[l], idx=self.idx[l], g=self.g[l], stream=main)
            if self.fused:
                self.base[l].gemv_unmerged((self.idx[s][0], self.g[s][0]), stream=main)
                continue
            if side is not None:
                fork, join = self._ev[l]
                fork.record(main)
                side.wait_event(fork)
            # the adapters are enqueued first, so their few workgroups are
            # dispatched before the base product fills the machine
            if self.grouped:
                self.groups[l].run(self.idx[s], self.g[s], workspace=self.ws, stream=ad)
            else:
                for (W, A, B), x, y in zip(projs, self.xs[l], self.y_lora[l]):
                    sgmm(x[None], self.idx[s], self.g[s], A, B, y, self.scale, workspace=self.ws,
                         stream=ad)
            self.base[l].gemv(stream=main)
            if side is not None:
                join.record(side)
                main.wait_event(join)

    def reset_lora(self):
        """Zero the adapter outputs (they accumulate across tokens; the fused
        form overwrites its outputs and has none)."""
        for yl in self.y_lora:
            for y in yl:
                y.zero_()

    def launches_per_token(self) -> int:
        """Kernel launches one step() makes: the router (once per layer, or once
        per token with route_once), per layer the base product (dlm_gemv: 1) and
        the adapters' SGMM launches, or with fused the layer's dlm_gemv_unmerged
        launches."""
        n = 1 if self.route_once else len(self.projs)
        for l, projs in enumerate(self.projs):
            if self.fused:
                n += self.base[l].launches_per_gemv_unmerged()
                continue
            if self.grouped:
                sg = sgmm_launches(1, max(W.shape[1] for W, _, _ in projs), self.r, len(projs), self.dtype)
            else:
                sg = sum(sgmm_launches(1, W.shape[1], self.r, 1, self.dtype) for W, _, _ in projs)
            n += 1 + sg
        return n

    def status(self, stream=None) -> int:
        """DLM_OK, or the first failure the device reported (sets, weights)."""
        s = DLM_OK if self.ws is None else sgmm_status(self.ws, stream)
        if s != DLM_OK:
            return s
        for h in self.base:
            s = h.status(stream)
            if s != DLM_OK:
                return s
        return DLM_OK

    def close(self):
        for h in self.base:
            h.close()
        for grp in self.groups:
            grp.close()
        self.base, self.groups = [], []


__all__ = ["LayerwiseDecode"]
