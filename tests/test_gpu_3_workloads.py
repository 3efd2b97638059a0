"""The standard workloads at full size, in the launch configuration the
benchmark times (AUTO mode, add into y): sampled rows against the oracle, plus
the invariants that hold at any size."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DevCase, check_rows, from_dev, oracle_rows, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6])
def test_workload_parity(L, k):
    c = W.config(k)
    print(f"[workload] {c.name} T={c.T}", flush=True)
    d = DevCase(c)
    y, meta = d.apply(L, mode="auto", add=True)
    rows = np.arange(c.T) if c.T <= 256 else sample_rows(c)
    idx = torch.from_numpy(rows).cuda()
    got = from_dev(y.index_select(0, idx))
    ref = oracle_rows(c, rows)
    err = check_rows(c, got, ref, c.name)
    print(f"[workload] {c.name}: {rows.shape[0]} rows checked, max rel err {err:.3e}", flush=True)
    # rows without an adapter are bit-identical to the base output
    none = np.where(c.token_slot < 0)[0]
    if none.size:
        ni = torch.from_numpy(none).cuda()
        assert torch.equal(y.index_select(0, ni), d.y0.index_select(0, ni))
    del y, d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k,mode", [(2, "bgmv"), (2, "sgmv"), (3, "bgmv"), (4, "sgmv"), (5, "bgmv"), (5, "sgmv"),
                                    (6, "bgmv"), (6, "sgmv")])
def test_workload_modes(L, k, mode):
    c = W.config(k)
    print(f"[workload-mode] {c.name} mode={mode}", flush=True)
    d = DevCase(c)
    y, _ = d.apply(L, mode=mode, add=True)
    rows = sample_rows(c, k_random=48, seed=k)
    got = from_dev(y.index_select(0, torch.from_numpy(rows).cuda()))
    check_rows(c, got, oracle_rows(c, rows), f"{c.name}/{mode}")
    del y, d
    torch.cuda.empty_cache()


def test_toy_full_forward(L):
    """The handbook toy end to end: base product by torch on the device, the
    delta by the library, against the oracle's fp64 x*W + delta (all rows)."""
    c = W.config(1)
    d = DevCase(c)
    Wd = torch.from_numpy(c.notes["W"]).cuda()
    y = d.x @ Wd
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    L.lora_apply(meta, d.x, d.A, d.B, c.offsets, y, scale=c.scale)
    zero = np.zeros_like(c.y0)
    import oracle
    ref = oracle.lora_rows(c.x, c.token_slot, c.num_slots, c.A, c.B, [0], c.scale, zero) + \
        c.x.astype(np.float64) @ c.notes["W"].astype(np.float64)
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-4 * (1 + np.abs(ref)))


def test_logits_rows_through_the_sampler_mapping(L):
    """The vocabulary-projection LoRA on sampled rows: gather the sampler's rows
    of a full step's hidden states, build the metadata from the sampler-side
    slot list, and compare every sampled row with the oracle."""
    c = W.config(6)
    step_lengths = c.notes["step_lengths"]
    rows = c.notes["sampled_token_rows"]
    # a full step of hidden states whose sampled rows are the workload's x
    T_step = int(step_lengths.sum())
    full = torch.zeros((T_step, c.d_in), dtype=torch.bfloat16, device="cuda")
    d = DevCase(c)
    full[torch.from_numpy(rows).cuda()] = d.x
    xs = full.index_select(0, torch.from_numpy(rows).cuda())
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    L.lora_apply(meta, xs, d.A, d.B, c.offsets, y, scale=c.scale)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), "logits, all sampled rows")
