"""Host-side checks of the layer-wise composition (no GPU): the launch count it
reports is the sum of the library's own per-call counts, and mismatched
argument lists are refused before anything touches a device."""
import pytest
import torch

import dynamic_lora_moe_amd as dlm
from dynamic_lora_moe_amd.layerwise import LayerwiseDecode


class _W:
    """Stands in for a weight in the launch arithmetic (only .shape is read)."""

    def __init__(self, d_out, d_in):
        self.shape = (d_out, d_in)


class _Handle:
    """Stands in for a layer handle in the launch arithmetic of the fused form."""

    def launches_per_gemv_unmerged(self):
        return 2


def _fake(projs, route_once, grouped, fused=False):
    lw = LayerwiseDecode.__new__(LayerwiseDecode)
    lw.projs = projs
    lw.route_once, lw.grouped, lw.fused = route_once, grouped, fused
    lw.base = [_Handle() for _ in projs]
    lw.r = 16
    lw.dtype = torch.bfloat16
    return lw


@pytest.mark.parametrize("route_once", [False, True])
@pytest.mark.parametrize("grouped", [False, True])
def test_launches_per_token_adds_the_library_counts(route_once, grouped):
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    layers = [[(_W(o, i), None, None) for o, i in shapes] for _ in range(3)]
    lw = _fake(layers, route_once, grouped)
    per_layer = (dlm.sgmm_launches(1, 11008, 16, len(shapes)) if grouped
                 else sum(dlm.sgmm_launches(1, i, 16, 1) for _, i in shapes))
    routers = 1 if route_once else len(layers)
    assert lw.launches_per_token() == routers + len(layers) * (1 + per_layer)


@pytest.mark.parametrize("route_once", [False, True])
def test_fused_launches_are_the_routers_and_two_per_layer(route_once):
    layers = [[(_W(4096, 4096), None, None)] * 7 for _ in range(5)]
    lw = _fake(layers, route_once, False, fused=True)
    assert lw.launches_per_token() == (1 if route_once else 5) + 5 * 2


def test_fused_with_grouped_is_refused():
    with pytest.raises(ValueError):
        LayerwiseDecode([[]], [None], [[]], 8, 16, 2.0, grouped=True, fused=True)


def test_mismatched_lists_are_refused():
    with pytest.raises(ValueError):
        LayerwiseDecode([[]], [], [[]], 8, 16, 2.0)
    with pytest.raises(ValueError):
        LayerwiseDecode([[], []], [None, None], [[]], 8, 16, 2.0)
