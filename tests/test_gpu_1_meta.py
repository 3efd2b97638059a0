"""GPU slot metadata against the oracle: bit-exact on every array.  Batches of
8192 rows and more are counted in parts by several workgroups (up to 64 parts
of at least 1024 rows, a part taking 1024 rows per step); smaller ones run on
one workgroup, which from 3072 rows scatters batches of mixed keys through LDS
(the random, Zipf and bad-id patterns) and the others straight to memory
(sorted, reversed, one slot, all without an adapter)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def _meta_check(L, ts_np, S, label):
    print(f"[meta] {label} T={ts_np.shape[0]} S={S}", flush=True)
    ts = torch.from_numpy(np.ascontiguousarray(ts_np, np.int32)).cuda()
    m = L.lora_prepare_meta(ts, S)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in m.tensors().items()}
    ref = oracle.prepare_meta(ts_np, S)
    assert np.array_equal(got["sorted"], ref.sorted), label
    eff = np.where((ts_np >= -1) & (ts_np < S), ts_np, -1)
    assert np.array_equal(got["sorted_slot"], eff[ref.sorted]), label
    assert np.array_equal(got["seg_slot"], ref.seg_slot), label
    assert np.array_equal(got["seg_count"], ref.seg_count), label
    assert np.array_equal(got["seg_start"], ref.seg_start), label
    info = got["info"]
    assert info[0] == ref.num_segments and info[1] == ref.no_lora and info[2] == ref.num_bad, label
    assert info[3] == int(np.sum((ts_np < -1) | (ts_np >= S) | (ts_np == -1))), label
    # work tiles: every segment of the oracle's metadata cut into runs of 64
    # sorted positions, in order (the library's own tile format)
    tiles = got["tiles"]
    k = 0
    for g in range(ref.num_segments):
        slot, c, st = int(ref.seg_slot[g]), int(ref.seg_count[g]), int(ref.seg_start[g])
        for i in range((c + 63) // 64):
            rows, pos0 = min(64, c - 64 * i), st + 64 * i
            assert list(tiles[k, :4]) == [slot, rows, pos0, 0], (label, k)
            assert np.array_equal(tiles[k, 4:4 + rows], ref.sorted[pos0:pos0 + rows]), (label, k)
            k += 1
    assert info[4] == k and list(info[5:8]) == [0, 0, 0], label
    assert k <= L.max_tiles(ts_np.shape[0], S), label


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_meta_workloads(L, k):
    c = W.config(k)
    _meta_check(L, c.token_slot, c.num_slots, c.name)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


PATTERNS = ["uniform", "all_none", "one_slot", "sorted", "reversed", "zipf", "bad_ids"]


@pytest.mark.parametrize("T", [0, 1, 2, 63, 64, 65, 1023, 1024, 1025, 3071, 3072, 5000, 8191, 8192, 20000])
@pytest.mark.parametrize("S", [1, 2, 33, 128, 1023])
@pytest.mark.parametrize("pattern", PATTERNS)
def test_meta_random(L, T, S, pattern):
    rng = _rng(T * 7919 + S * 31 + PATTERNS.index(pattern))
    if pattern == "uniform":
        ts = rng.integers(-1, S, T)
    elif pattern == "all_none":
        ts = np.full(T, -1)
    elif pattern == "one_slot":
        ts = np.full(T, S - 1)
    elif pattern == "sorted":
        ts = np.sort(rng.integers(-1, S, T))
    elif pattern == "reversed":
        ts = np.sort(rng.integers(-1, S, T))[::-1]
    elif pattern == "zipf":
        ts = W.zipf_slots(rng, T, S, 1.1) if T else np.zeros(0, int)
    else:
        ts = rng.integers(-3, S + 3, T)
    _meta_check(L, ts.astype(np.int32), S, f"{pattern}")


def test_meta_repeatable_and_workspace_reuse(L):
    """Same input twice into one workspace: identical arrays (no stale state)."""
    rng = _rng(5)
    ts_np = rng.integers(-1, 64, 4000).astype(np.int32)
    ts = torch.from_numpy(ts_np).cuda()
    ws = torch.full((L.lora_meta_workspace_bytes(4000, 64),), 0x5A, dtype=torch.uint8, device="cuda")
    a = {k: v.clone() for k, v in L.lora_prepare_meta(ts, 64, workspace=ws).tensors().items()}
    other = torch.from_numpy(rng.integers(-1, 64, 4000).astype(np.int32)).cuda()
    L.lora_prepare_meta(other, 64, workspace=ws)
    b = L.lora_prepare_meta(ts, 64, workspace=ws).tensors()
    torch.cuda.synchronize()
    for k in a:
        if k != "tiles":
            assert torch.equal(a[k], b[k]), k
    # tiles: the defined part (headers and the rows token indices of each tile)
    ta, tb = a["tiles"].cpu().numpy(), b["tiles"].cpu().numpy()
    for i in range(int(a["info"][4])):
        rows = int(ta[i, 1])
        assert np.array_equal(ta[i, :4 + rows], tb[i, :4 + rows]), i


@pytest.mark.parametrize("S", [8, 1023])
@pytest.mark.parametrize("pattern", ["uniform", "zipf", "bad_ids"])
def test_meta_many_parts(L, S, pattern):
    """100 000 rows: 64 parts of 1563 rows, each two steps of up to 1024."""
    T = 100_000
    rng = _rng(S * 17 + PATTERNS.index(pattern))
    if pattern == "uniform":
        ts = rng.integers(-1, S, T)
    elif pattern == "zipf":
        ts = W.zipf_slots(rng, T, S, 1.1)
    else:
        ts = rng.integers(-3, S + 3, T)
    _meta_check(L, ts.astype(np.int32), S, f"many parts {pattern}")


def test_meta_parts_repeatable_and_workspace_reuse(L):
    """The several-workgroup path twice into one workspace, another batch in
    between: identical arrays (its counts are rebuilt on every call)."""
    rng = _rng(6)
    ts_np = rng.integers(-1, 64, 9000).astype(np.int32)
    ts = torch.from_numpy(ts_np).cuda()
    ws = torch.full((L.lora_meta_workspace_bytes(9000, 64),), 0x5A, dtype=torch.uint8, device="cuda")
    a = {k: v.clone() for k, v in L.lora_prepare_meta(ts, 64, workspace=ws).tensors().items()}
    other = torch.from_numpy(rng.integers(-1, 64, 9000).astype(np.int32)).cuda()
    L.lora_prepare_meta(other, 64, workspace=ws)
    b = L.lora_prepare_meta(ts, 64, workspace=ws).tensors()
    torch.cuda.synchronize()
    for k in a:
        if k != "tiles":
            assert torch.equal(a[k], b[k]), k
    ta, tb = a["tiles"].cpu().numpy(), b["tiles"].cpu().numpy()
    for i in range(int(a["info"][4])):
        rows = int(ta[i, 1])
        assert np.array_equal(ta[i, :4 + rows], tb[i, :4 + rows]), i
    _meta_check(L, ts_np, 64, "parts, checked against the oracle")
