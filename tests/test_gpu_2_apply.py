"""GPU shrink / expand / apply against the oracle on every row of small batches
that still span several tiles and ragged tails: ranks 8..64, fp32 and bf16,
the three modes, add and store, unequal slices with gaps in y."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DELTA_L2, DevCase, as_f64, check_rows, from_dev, oracle_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def small_case(seed, dtype, r, S=7, with_none=True):
    """Mixed batch: one-token requests, segments just below/above the 64-row
    matrix tile and the 16-token path threshold, a 3-slice output with gaps."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.array([1] * 24 + [3, 70, 5, 130, 17, 64, 65, 1, 200, 15, 16, 9], np.int64)
    req = rng.integers(-1 if with_none else 0, S, lengths.shape[0]).astype(np.int32)
    req[-5] = S - 1
    ranks = np.minimum(r, rng.choice(np.array([r, max(1, r // 2), max(1, r // 4)]), S)).astype(np.int32)
    c = W.make_case(name=f"small_{dtype}_r{r}", seed=seed, rng=rng, dtype=dtype, lengths=lengths,
                    req_slot=req, num_slots=S, d_in=264, r_max=r, widths=[136, 72, 40],
                    offsets=[0, 144, 224], ldy=272, scale=0.75, ranks=ranks, weight_sd=0.05)
    c.slot_scale = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), S)
    return c


def _bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("r", [8, 16, 32, 64])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
@pytest.mark.parametrize("add", [True, False])
def test_apply_small_all_rows(L, dtype, r, mode, add):
    c = small_case(100 + r, dtype, r)
    print(f"[apply] {c.name} T={c.T} mode={mode} add={add}", flush=True)
    d = DevCase(c)
    y, _ = d.apply(L, mode=mode, add=add)
    got = from_dev(y)
    ref = oracle_rows(c, np.arange(c.T), add=add)
    check_rows(c, got, ref, c.name)
    # never-written positions are bit-identical to the input
    outside = np.ones(c.ldy, bool)
    for w, o in zip(c.widths, c.offsets):
        outside[o:o + w] = False
    assert _bits_equal(got[:, outside], c.y0[:, outside])
    none = c.token_slot < 0
    assert none.any()
    if add:
        assert _bits_equal(got[none], c.y0[none])
    else:
        inside = ~outside
        assert np.all(as_f64(got[none][:, inside]) == 0)
        # relative L2 of the delta (the windows hold the delta itself)
        dg, dr = as_f64(got[:, inside]), ref[:, inside]
        assert np.linalg.norm(dg - dr) <= DELTA_L2[dtype] * np.linalg.norm(dr)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("r", [16, 64])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_shrink_alone(L, dtype, r, mode):
    c = small_case(200 + r, dtype, r)
    print(f"[shrink] {c.name} mode={mode}", flush=True)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    u = torch.full((c.n_slices, c.T, r), float("nan"), dtype=torch.float32, device="cuda")
    L.lora_shrink(meta, d.x, d.A, u, scale=c.scale, slot_scale=d.slot_scale, mode=mode)
    got = u.cpu().numpy()
    _, uref = oracle_rows(c, np.arange(c.T), return_u=True)     # [T][n_slices][r]
    lora = c.token_slot >= 0
    for s in range(c.n_slices):
        g, rf = got[s][lora].astype(np.float64), uref[lora, s]
        assert np.all(np.abs(g - rf) <= 1e-4 * (1 + np.abs(rf))), (s, np.max(np.abs(g - rf)))
    assert np.all(np.isnan(got[:, ~lora]))       # rows without an adapter are not written


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("r", [8, 32, 64])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
@pytest.mark.parametrize("add", [True, False])
def test_expand_alone(L, dtype, r, mode, add):
    """Expand from a seeded fp32 rank-r buffer (drawn by the input generator,
    so neither side consumes a result of the other)."""
    c = small_case(300 + r, dtype, r)
    print(f"[expand] {c.name} mode={mode} add={add}", flush=True)
    rng = np.random.Generator(np.random.PCG64(7 + r))
    u_np = rng.standard_normal((c.n_slices, c.T, r), dtype=np.float32)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    L.lora_expand(meta, torch.from_numpy(u_np).cuda(), d.B, c.offsets, y, add=add, mode=mode)
    ref = oracle.expand_rows(u_np, c.token_slot, c.num_slots, c.B, c.offsets, c.y0, add=add)
    check_rows(c, from_dev(y), ref, c.name)


def test_modes_agree(L):
    """BGMV, SGMV and AUTO give the same y within the bf16 gate, and each is
    deterministic run to run."""
    c = small_case(400, "bf16", 32)
    d = DevCase(c)
    outs = {}
    for mode in ("bgmv", "sgmv", "auto"):
        a = from_dev(d.apply(L, mode=mode)[0])
        b = from_dev(d.apply(L, mode=mode)[0])
        assert np.array_equal(a, b), mode
        outs[mode] = as_f64(a)
    ref = oracle_rows(c, np.arange(c.T))
    for m, v in outs.items():
        assert np.all(np.abs(v - ref) <= 2e-2 * (1 + np.abs(ref))), m


def many_slices_case(seed, dtype, r, n_slices=8):
    """Eight packed slices of uneven widths with gaps between windows: the
    matrix-core shrink covers the slices' ranks in one or two passes of output
    columns, and the expand walks many (slice, column chunk) pairs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.array([1] * 10 + [40, 2, 90, 17, 1, 66], np.int64)
    S = 5
    req = rng.integers(-1, S, lengths.shape[0]).astype(np.int32)
    widths = [24, 136, 8, 64, 200, 40, 16, 128][:n_slices]
    offsets, o = [], 0
    for w in widths:
        offsets.append(o)
        o += w + 8
    c = W.make_case(name=f"slices{n_slices}_{dtype}_r{r}", seed=seed, rng=rng, dtype=dtype,
                    lengths=lengths, req_slot=req, num_slots=S, d_in=392, r_max=r, widths=widths,
                    offsets=offsets, ldy=o, scale=1.25, weight_sd=0.05)
    return c


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("r", [8, 16, 32, 64])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_apply_many_slices(L, dtype, r, mode):
    c = many_slices_case(300 + r, dtype, r)
    print(f"[slices] {c.name} T={c.T} mode={mode}", flush=True)
    d = DevCase(c)
    for add in (True, False):
        y, _ = d.apply(L, mode=mode, add=add)
        got = from_dev(y)
        check_rows(c, got, oracle_rows(c, np.arange(c.T), add=add), f"{c.name} add={add}")
        outside = np.ones(c.ldy, bool)
        for w, o in zip(c.widths, c.offsets):
            outside[o:o + w] = False
        assert _bits_equal(got[:, outside], c.y0[:, outside])
