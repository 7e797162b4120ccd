"""The per-call entry points allocate no device memory: free device memory
(hipMemGetInfo, through torch) is the same before and after many calls of the
router, the switch (rank 16 and the rank-64 path with its packed A copy), the
fused switch + product and the SGMM (single and grouped), once handles,
workspaces and sets exist."""
import numpy as np
import pytest
import torch

import dynamic_lora_moe_amd as dlm
import synth

pytestmark = pytest.mark.gpu


def _bank(d_out, d_in, E, r, key):
    dt = torch.bfloat16
    return (synth.normal_device((d_out, d_in), 0.02, dt, "cuda", "mem", key, "W"),
            synth.normal_device((E, r, d_in), 0.02, dt, "cuda", "mem", key, "A"),
            synth.normal_device((E, d_out, r), 0.02, dt, "cuda", "mem", key, "B"))


def test_per_call_entry_points_allocate_nothing():
    E, T = 8, 300
    L16 = dlm.Layers([_bank(512, 256, E, 16, 0), _bank(264, 512, E, 16, 1)], E, 16, 2.0)
    L64 = dlm.Layers([_bank(512, 4096, E, 64, 2), _bank(300, 520, E, 64, 3)], E, 64, 1.0)
    xs = [torch.randn(256, device="cuda").bfloat16(), torch.randn(512, device="cuda").bfloat16()]
    ys = [torch.empty(512, device="cuda"), torch.empty(264, device="cuda")]
    L16.bind_vectors(xs, ys)
    sets = [(torch.tensor([i, (i + 3) % E], dtype=torch.int32, device="cuda"),
             torch.tensor([0.7, 0.3], device="cuda")) for i in range(4)]
    xr = torch.randn(T, 256, device="cuda").bfloat16()
    Wr = (0.02 * torch.randn(256, E, device="cuda")).bfloat16()
    idx = torch.empty(T, 2, dtype=torch.int32, device="cuda")
    g = torch.empty(T, 2, device="cuda")
    probs = [(torch.randn(T, 256, device="cuda").bfloat16(), *[t for t in _bank(136, 256, E, 16, 4)[1:]],
              torch.zeros(T, 136, device="cuda").bfloat16()),
             (torch.randn(T, 1040, device="cuda").bfloat16(), *[t for t in _bank(64, 1040, E, 16, 5)[1:]],
              torch.zeros(T, 64, device="cuda").bfloat16())]
    grp = dlm.SgmmGroup(probs, E, 16, 1.0)
    ws = grp.workspace(T)
    x1, A1, B1, y1 = probs[0]
    ws1 = dlm.sgmm_workspace(T, 256, E, 16)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for i in range(6):
        dlm.pregate(xr, Wr, idx, g)
        L16.switch(sets[i % 4], sets[(i + 1) % 4])
        L64.switch(sets[i % 4], sets[(i + 1) % 4])
        L16.switch_gemv(sets[(i + 1) % 4], sets[i % 4])
        L16.gemv()
        grp.run(idx, g, workspace=ws)
        dlm.sgmm(x1, idx, g, A1, B1, y1, 1.0, ws1)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)
    assert L16.status() == dlm.DLM_OK and L64.status() == dlm.DLM_OK
    assert dlm.sgmm_status(ws) == dlm.DLM_OK and dlm.sgmm_status(ws1) == dlm.DLM_OK
    for h in (L16, L64, grp):
        h.close()
