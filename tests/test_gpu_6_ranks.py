"""Per-slot ranks (d_slot_rank): the kernels read only the ranks each slot's
adapter really has (rounded up to 8), so padding past them is never touched.
The tests fill that padding with NaN: a kernel that reads it turns its output
into NaN.  The oracle runs on the zero-padded factors, whose result is the
defined one (a slot's buffers hold zeros past its rank)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DELTA_L2, DevCase, as_f64, check_rows, from_dev, oracle_rows, to_dev
from test_gpu_2_apply import small_case
from test_gpu_4_edges import integer_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def nan_padded(c):
    """Copies of A and B whose entries past each slot's rank rounded up to 8
    are NaN (between the rank and that bound they stay zero)."""
    nan = W.bf16_round(np.array([np.nan], np.float32))[0] if c.dtype == "bf16" else np.float32(np.nan)
    A, B = [], []
    for a, b in zip(c.A, c.B):
        a, b = a.copy(), b.copy()
        for slot in range(c.num_slots):
            r8 = min(c.r_max, (int(c.ranks[slot]) + 7) // 8 * 8)
            a[slot, :, r8:] = nan
            b[slot, r8:, :] = nan
        A.append(a)
        B.append(b)
    return A, B


class RankedDev(DevCase):
    def __init__(self, c):
        super().__init__(c)
        A, B = nan_padded(c)
        self.A = [to_dev(a, c.dtype) for a in A]
        self.B = [to_dev(b, c.dtype) for b in B]
        self.ranks = torch.from_numpy(np.asarray(c.ranks, np.int32)).cuda()

    def apply_ranked(self, L, mode="auto", add=True):
        meta = L.lora_prepare_meta(self.token_slot, self.c.num_slots)
        y = self.y0.clone()
        L.lora_apply(meta, self.x, self.A, self.B, self.c.offsets, y, scale=self.c.scale,
                     slot_scale=self.slot_scale, add=add, mode=mode, slot_rank=self.ranks)
        return y, meta


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("r", [8, 16, 32, 64])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_ranked_apply_small(L, dtype, r, mode):
    c = small_case(500 + r, dtype, r)
    print(f"[ranks] {c.name} ranks={sorted(set(c.ranks.tolist()))} mode={mode}", flush=True)
    d = RankedDev(c)
    for add in (True, False):
        y, _ = d.apply_ranked(L, mode=mode, add=add)
        got = from_dev(y)
        check_rows(c, got, oracle_rows(c, np.arange(c.T), add=add), f"{c.name} add={add}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["auto", "sgmv"])
def test_ranked_shrink_and_expand_alone(L, dtype, mode):
    c = small_case(600, dtype, 64)
    d = RankedDev(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    u = torch.full((c.n_slices, c.T, c.r_max), float("nan"), dtype=torch.float32, device="cuda")
    L.lora_shrink(meta, d.x, d.A, u, scale=c.scale, slot_scale=d.slot_scale, mode=mode, slot_rank=d.ranks)
    torch.cuda.synchronize()
    _, uref = oracle_rows(c, np.arange(c.T), return_u=True)
    got = u.cpu().numpy()
    has = c.token_slot >= 0
    for s in range(c.n_slices):
        g = got[s][has].astype(np.float64)
        ref = uref[has, s, :]
        tol = 1e-4 if dtype == "f32" else 2e-2
        assert np.all(np.abs(g - ref) <= tol * (1 + np.abs(ref))), s
        # ranks past each token's slot rank are written as exact zeros
        r8 = np.minimum(c.r_max, (c.ranks[c.token_slot[has]] + 7) // 8 * 8)
        for i in range(g.shape[0]):
            assert np.all(g[i, r8[i]:] == 0.0)
    # the expand alone, from the oracle's u (zeros past the ranks)
    y = d.y0.clone()
    uu = torch.from_numpy(np.ascontiguousarray(np.transpose(uref, (1, 0, 2))).astype(np.float32)).cuda()
    uu[:, ~torch.from_numpy(has).cuda(), :] = 0
    L.lora_expand(meta, uu, d.B, c.offsets, y, add=True, mode=mode, slot_rank=d.ranks)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), "expand alone")


@pytest.mark.parametrize("k", [4, 5])
@pytest.mark.parametrize("mode", ["auto", "bgmv"])
def test_ranked_workloads(L, k, mode):
    """The mixed-rank workloads at full size, sampled rows."""
    c = W.config(k)
    print(f"[ranks] workload {c.name} mode={mode}", flush=True)
    d = RankedDev(c)
    y, _ = d.apply_ranked(L, mode=mode)
    rng = np.random.Generator(np.random.PCG64(k))
    rows = np.sort(rng.choice(c.T, 96, replace=False))
    check_rows(c, from_dev(y)[rows], oracle_rows(c, rows), c.name)


@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_ranked_integer_bit_exact(L, mode):
    c = integer_case(21, [1] * 200 + [300, 77], 16, 2048, [1024, 512], 64, 2.0)
    c.ranks = np.random.Generator(np.random.PCG64(3)).choice(np.array([8, 16, 32, 64], np.int32), 16)
    for a, b in zip(c.A, c.B):   # zero the factors past each slot's rank (the defined padding)
        for slot in range(16):
            a[slot, :, c.ranks[slot]:] = 0
            b[slot, c.ranks[slot]:, :] = 0
    ref = oracle_rows(c, np.arange(c.T))
    assert np.all(ref == np.round(ref)) and np.max(np.abs(ref)) <= 256
    d = RankedDev(c)
    y, _ = d.apply_ranked(L, mode=mode)
    assert np.array_equal(as_f64(from_dev(y)), ref)


# r_max that is not a power of two, and 128: A is [d_in][r_max] and B
# [r_max][width] per slot, packed at that rank; the kernels run at the next of
# 8, 16, 32, 64, 128 and must neither read past r_max into the next row nor
# let ranks past it add anything.

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("r", [24, 48, 128])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_apply_any_r_max(L, dtype, r, mode):
    c = small_case(700 + r, dtype, r)
    print(f"[r_max] {c.name} ranks={sorted(set(c.ranks.tolist()))} mode={mode}", flush=True)
    d = RankedDev(c)
    for add in (True, False):
        y, _ = d.apply_ranked(L, mode=mode, add=add)
        check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T), add=add), f"{c.name} ranked add={add}")
    plain = DevCase(c)                  # no d_slot_rank: every slot read at r_max
    y, _ = plain.apply(L, mode=mode, add=True)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), f"{c.name} r_max")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("r", [24, 40, 120])
def test_shrink_and_expand_alone_any_r_max(L, dtype, r):
    """lora_shrink writes the caller's u as [n_slices][T][r_max] and
    lora_expand reads it so, at a rank between the kernels' tile ranks."""
    c = small_case(800 + r, dtype, r)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    u = torch.full((c.n_slices, c.T, c.r_max), float("nan"), dtype=torch.float32, device="cuda")
    L.lora_shrink(meta, d.x, d.A, u, scale=c.scale, slot_scale=d.slot_scale, mode="auto")
    torch.cuda.synchronize()
    _, uref = oracle_rows(c, np.arange(c.T), return_u=True)
    got = u.cpu().numpy()
    has = c.token_slot >= 0
    tol = 1e-4 if dtype == "f32" else 2e-2
    for s in range(c.n_slices):
        g, ref = got[s][has].astype(np.float64), uref[has, s, :]
        assert np.all(np.abs(g - ref) <= tol * (1 + np.abs(ref))), s
    y = d.y0.clone()
    uu = torch.from_numpy(np.ascontiguousarray(np.transpose(uref, (1, 0, 2))).astype(np.float32)).cuda()
    uu[:, ~torch.from_numpy(has).cuda(), :] = 0
    L.lora_expand(meta, uu, d.B, c.offsets, y, add=True, mode="auto")
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), f"{c.name} expand alone")


@pytest.mark.parametrize("r", [24, 48, 128])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_any_r_max_integer_bit_exact(L, r, mode):
    """Integer inputs at r_max 24, 48 and 128 over long segments (the shrink's
    split of d_in and the long-segment expand) and one-token requests: every
    element bit-identical to the oracle."""
    c = integer_case(30 + r, [1] * 96 + [700, 300, 129, 64], 6, 2048, [1024, 512], r, 2.0)
    ref = oracle_rows(c, np.arange(c.T))
    assert np.all(ref == np.round(ref)) and np.max(np.abs(ref)) <= 256
    print(f"[r_max] integer r={r} T={c.T} mode={mode}", flush=True)
    d = DevCase(c)
    y, _ = d.apply(L, mode=mode, add=True)
    assert np.array_equal(as_f64(from_dev(y)), ref)


# A in the rank-major layout ([S][r_max][d_in], the pages' A layout): a slot's
# ranks are whole rows, so with per-slot ranks the rows past a slot's rank
# (rounded up to 8) are never fetched; the tests put NaN there.

def rank_rows(A, dtype):
    """Device copies of A [S][d_in][r] as [S][r][d_in]."""
    return [to_dev(np.ascontiguousarray(np.transpose(a, (0, 2, 1))), dtype) for a in A]


@pytest.mark.parametrize("r", [16, 24, 64, 128])
@pytest.mark.parametrize("mode", ["auto", "sgmv"])
def test_rank_rows_apply(L, r, mode):
    c = small_case(900 + r, "bf16", r)
    print(f"[rank-rows] {c.name} mode={mode}", flush=True)
    d = RankedDev(c)
    A_nan, _ = nan_padded(c)
    Arm = rank_rows(A_nan, c.dtype)
    for add in (True, False):
        meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
        y = d.y0.clone()
        L.lora_apply(meta, d.x, Arm, d.B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale, add=add, mode=mode,
                     slot_rank=d.ranks, a_rank_rows=True)
        check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T), add=add), f"{c.name} rank rows add={add}")
    # without per-slot ranks every rank row is read: the zero padding, no NaN
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    L.lora_apply(meta, d.x, rank_rows(c.A, c.dtype), d.B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale,
                 mode=mode, a_rank_rows=True)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), f"{c.name} rank rows, r_max read")


def test_rank_rows_shrink_alone_and_bgmv_refused(L):
    c = small_case(960, "bf16", 32)
    d = RankedDev(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    u = torch.full((c.n_slices, c.T, c.r_max), float("nan"), dtype=torch.float32, device="cuda")
    A_nan, _ = nan_padded(c)
    L.lora_shrink(meta, d.x, rank_rows(A_nan, c.dtype), u, scale=c.scale, slot_scale=d.slot_scale, mode="auto",
                  slot_rank=d.ranks, a_rank_rows=True)
    torch.cuda.synchronize()
    _, uref = oracle_rows(c, np.arange(c.T), return_u=True)
    got = u.cpu().numpy()
    has = c.token_slot >= 0
    for s in range(c.n_slices):
        g, ref = got[s][has].astype(np.float64), uref[has, s, :]
        assert np.all(np.abs(g - ref) <= 2e-2 * (1 + np.abs(ref))), s
    with pytest.raises(L.LoraError):
        L.lora_apply(meta, d.x, rank_rows(c.A, c.dtype), d.B, c.offsets, d.y0.clone(), scale=c.scale, mode="bgmv",
                     a_rank_rows=True)


@pytest.mark.parametrize("r", [32, 64])
def test_rank_rows_integer_bit_exact(L, r):
    c = integer_case(70 + r, [1] * 96 + [700, 300, 129, 64], 6, 2048, [1024, 512], r, 2.0)
    ref = oracle_rows(c, np.arange(c.T))
    assert np.all(ref == np.round(ref)) and np.max(np.abs(ref)) <= 256
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    for mode in ("auto", "sgmv"):
        y = d.y0.clone()
        L.lora_apply(meta, d.x, rank_rows(c.A, c.dtype), d.B, c.offsets, y, scale=c.scale, mode=mode,
                     a_rank_rows=True)
        assert np.array_equal(as_f64(from_dev(y)), ref), mode


@pytest.mark.parametrize("k", [4, 5])
def test_rank_rows_workloads(L, k):
    """The mixed-rank workloads at full size with rank-major A and per-slot
    ranks (NaN past every slot's rank rows), sampled rows."""
    c = W.config(k)
    print(f"[rank-rows] workload {c.name}", flush=True)
    d = RankedDev(c)
    A_nan, _ = nan_padded(c)
    Arm = rank_rows(A_nan, c.dtype)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    L.lora_apply(meta, d.x, Arm, d.B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale, slot_rank=d.ranks,
                 a_rank_rows=True)
    rng = np.random.Generator(np.random.PCG64(k))
    rows = np.sort(rng.choice(c.T, 96, replace=False))
    check_rows(c, from_dev(y)[rows], oracle_rows(c, rows), c.name)
    del Arm, y, d
    torch.cuda.empty_cache()
