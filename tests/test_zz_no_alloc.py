"""lora_apply_noalloc, the entry point for callers that cannot allocate: the
library's own device scratch replaces the workspace.  Through the C ABI, its
output equals lora_apply's (the same kernels on the same inputs, so bit for
bit) and the oracle's within the bf16 tolerance, 2e-2·(1+|ref|), on calls in a row
whose second input is smaller than the first; a call too large for the
scratch is refused."""
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


def decode_case(seed, T=256, S=32, d_in=4096, widths=(4096,), r=16):
    rng = np.random.Generator(np.random.PCG64(seed))
    req = rng.integers(0, S, T).astype(np.int32)
    req[rng.random(T) < 0.1] = -1
    return W.make_case(name=f"noalloc_decode_{seed}", seed=seed, rng=rng, dtype="bf16",
                       lengths=np.ones(T, np.int64), req_slot=req, num_slots=S, d_in=d_in, r_max=r,
                       widths=list(widths), scale=2.0, weight_sd=0.05)


def run_both(L, c, rows):
    """lora_apply (its own zeroed workspace) and lora_apply_noalloc on the same
    inputs: equal bits, and the oracle's rows within tolerance."""
    d = DevCase(c)
    y_ref, meta = d.apply(L, mode="auto", add=True)
    y = d.y0.clone()
    L.lora_apply_noalloc(meta, d.x, d.A, d.B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale, add=True)
    torch.cuda.synchronize()
    got, want = from_dev(y), from_dev(y_ref)
    assert np.array_equal(got.view(np.uint16) if got.dtype == np.uint16 else got.view(np.uint32),
                          want.view(np.uint16) if want.dtype == np.uint16 else want.view(np.uint32)), c.name
    check_rows(c, got[rows], oracle_rows(c, rows), c.name)


def test_noalloc_matches_apply_two_calls_second_smaller(L):
    """Workload 4 (mixed q/k/v, the shrink and expand tile kernels, 15 MiB of
    scratch), then a 256-token decode batch (the split kernel, whose
    rendezvous words live in the scratch), then that decode batch again."""
    big = W.config(4)
    print(f"[noalloc] {big.name} T={big.T}", flush=True)
    run_both(L, big, sample_rows(big))
    small = decode_case(710)
    for rep in range(2):
        print(f"[noalloc] {small.name} T={small.T} rep {rep}", flush=True)
        run_both(L, small, np.arange(small.T))


def test_noalloc_refuses_calls_beyond_the_scratch(L):
    """A call whose workspace would exceed the scratch is refused before any
    work is enqueued, and y is left as it was."""
    T, S, d_in, r = 65536, 8, 512, 64
    need = L.lora_apply_workspace_bytes(T, S, d_in, 4, r, torch.bfloat16)
    assert need > L.NOALLOC_SCRATCH_BYTES
    ts = torch.zeros(T, dtype=torch.int32, device="cuda")
    meta = L.lora_prepare_meta(ts, S)
    x = torch.zeros(T, d_in, dtype=torch.bfloat16, device="cuda")
    A = [torch.zeros(S, d_in, r, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    B = [torch.zeros(S, r, 32, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    y = torch.ones(T, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.LoraError) as e:
        L.lora_apply_noalloc(meta, x, A, B, [0, 32, 64, 96], y)
    assert e.value.status == L.LORA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 1).all())
