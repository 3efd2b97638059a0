"""Calls captured in a HIP graph: every replay, with eager work and
synchronisations between replays, gives the eager result bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DevCase, from_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


@pytest.mark.parametrize("k,mode", [(2, "auto"), (2, "sgmv"), (4, "auto"), (1, "auto")])
def test_graph_replays_match_eager(L, k, mode):
    c = W.config(k)
    print(f"[graph] {c.name} mode={mode}", flush=True)
    d = DevCase(c)
    ws = L.apply_workspace(L.lora_apply_workspace_bytes(c.T, c.num_slots, c.d_in, c.n_slices, c.r_max,
                                                        d.x.dtype, mode))
    mws = torch.empty(L.lora_meta_workspace_bytes(c.T, c.num_slots), dtype=torch.uint8, device="cuda")
    y = d.y0.clone()

    def call():
        meta = L.lora_prepare_meta(d.token_slot, c.num_slots, workspace=mws)
        L.lora_apply(meta, d.x, d.A, d.B, c.offsets, y, scale=c.scale, add=False, mode=mode,
                     workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = from_dev(y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        y.copy_(d.y0)            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(y), eager), f"replay {rep}"
