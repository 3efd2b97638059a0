"""Batches of long segments (a few hundred tokens per slot and more), the
shape of prefill: the matrix-core shrink with its k-chunks and the
long-segment expand.  Ragged k-chunks, several column groups of A, both A
layouts, per-slot ranks with NaN past them, slot scales, tokens without an
adapter, both y modes, one slot over thousands of tokens, and an integer case
that every summation order gets exactly."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DELTA_L2, DevCase, as_f64, check_rows, from_dev, oracle_rows
from test_gpu_4_edges import integer_case
from test_gpu_6_ranks import RankedDev, nan_padded, rank_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def long_case(seed, r, d_in, widths, S=3, ranks=True):
    """S slots, segments of 700, 300, 129 and 65 tokens plus one-token and
    no-adapter requests: at least 256 tokens per slot, tiles with ragged
    tails."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.array([700, 1, 300, 3, 129, 1, 65, 40, 513, 17], np.int64)
    req = np.array([0, 1, 1, -1, 2, 0, 0, -1, 2, 1], np.int32) % S
    req[[3, 7]] = -1
    rk = (np.minimum(r, rng.choice(np.array([r, max(8, r // 2), 8]), S)).astype(np.int32) if ranks
          else None)
    c = W.make_case(name=f"long_r{r}_d{d_in}_n{len(widths)}", seed=seed, rng=rng, dtype="bf16", lengths=lengths,
                    req_slot=req, num_slots=S, d_in=d_in, r_max=r, widths=widths, scale=0.5, ranks=rk,
                    weight_sd=0.05)
    c.slot_scale = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), S)
    assert c.T >= 256 * S
    return c


SHAPES = [
    # (r_max, d_in, widths): one slice; d_in off the k-tile size; three slices
    # of rank 64 side by side (192 shrink columns); r_max below the tile rank
    (16, 1000, [256]),
    (32, 2056, [512, 128, 128]),
    (64, 1024, [384, 256]),
    (64, 2312, [256, 128, 200]),
    (24, 1536, [264]),
    (48, 776, [136, 72]),
]


@pytest.mark.parametrize("r,d_in,widths", SHAPES)
@pytest.mark.parametrize("rank_major", [False, True])
def test_long_segments_ranked(L, r, d_in, widths, rank_major):
    c = long_case(1100 + r + d_in, r, d_in, widths)
    print(f"[long] {c.name} T={c.T} rank_major={rank_major}", flush=True)
    d = RankedDev(c)
    A_nan, _ = nan_padded(c)
    A = rank_rows(A_nan, c.dtype) if rank_major else d.A
    for add in (True, False):
        meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
        y = d.y0.clone()
        L.lora_apply(meta, d.x, A, d.B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale, add=add,
                     slot_rank=d.ranks, a_rank_rows=rank_major)
        got = from_dev(y)
        ref = oracle_rows(c, np.arange(c.T), add=add)
        check_rows(c, got, ref, f"{c.name} add={add}")
        if not add:  # the delta alone, relative to its own size
            err = np.linalg.norm(as_f64(got) - ref) / max(np.linalg.norm(ref), 1e-30)
            assert err <= DELTA_L2["bf16"], err


@pytest.mark.parametrize("r", [16, 32, 64])
def test_long_segments_integer_bit_exact(L, r):
    c = integer_case(1200 + r, [700, 300, 1, 129, 65, 513, 257], 3, 3080, [512, 256], r, 2.0)
    assert c.T >= 256 * 3
    print(f"[long-int] r={r} T={c.T}", flush=True)
    ref, u = oracle_rows(c, np.arange(c.T), return_u=True)
    assert np.max(np.abs(u)) <= 256 and np.max(np.abs(ref)) <= 256 and np.all(ref == np.round(ref))
    d = DevCase(c)
    for rank_major in (False, True):
        meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
        y = d.y0.clone()
        A = rank_rows(c.A, c.dtype) if rank_major else d.A
        L.lora_apply(meta, d.x, A, d.B, c.offsets, y, scale=c.scale, a_rank_rows=rank_major)
        assert np.array_equal(as_f64(from_dev(y)), ref), rank_major


def test_long_segments_one_slot_many_runs(L):
    """One slot, 5000 tokens: one segment cut into 79 tiles, the last one
    ragged."""
    rng = np.random.Generator(np.random.PCG64(1300))
    c = W.make_case(name="long_one_slot", seed=1300, rng=rng, dtype="bf16", lengths=np.array([4999, 1]),
                    req_slot=np.array([0, -1], np.int32), num_slots=1, d_in=4096, r_max=64, widths=[512],
                    weight_sd=0.05)
    d = DevCase(c)
    y, _ = d.apply(L)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), c.name)


def test_long_segments_workspace_is_enough(L):
    """A workspace of exactly the reported size, filled with garbage past the
    count words, gives the right result (d_in 4104: a ragged last k-chunk)."""
    c = long_case(1400, 64, 4104, [128])
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    need = L.lora_apply_workspace_bytes(c.T, c.num_slots, c.d_in, 1, 64, torch.bfloat16)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    L.lora_apply_workspace_init(ws)
    y, _ = d.apply(L, meta=meta, workspace=ws)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), c.name)
