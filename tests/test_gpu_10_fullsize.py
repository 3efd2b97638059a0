"""The standard workloads at full size in store mode (add = 0), where every
slice window of a row holds the delta itself, so the tolerance gate and the
relative L2 gate apply to the LoRA contribution at its real magnitude rather
than to y0 + delta; and integer-valued inputs at the exact batch plans of the
many-adapter decode workload (4096 tokens, 128 slots drawn Zipf(0.8), d_in
14336, rank 64) and of the prefill gate/up workload (17 705 tokens, d_in 4096,
two slices of 14 336 columns, rank 64), where every summation order is exact
and the library must match the oracle bit for bit.  Page "多 LoRA 服务：分段矩阵乘与
适配器调度", section "不合并权重，批量计算": every form of the batched product equals
the per-request result."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DELTA_L2, DevCase, as_f64, check_rows, from_dev, oracle_rows, sample_rows
from test_gpu_7_moe import MoeDev, moe_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def windows(c):
    inside = np.zeros(c.ldy, bool)
    for w, o in zip(c.widths, c.offsets):
        inside[o:o + w] = True
    return inside


def delta_gates(c, got, ref, what):
    """Store mode: element gate on the delta, relative L2 of the delta over the
    checked rows, and rows without an adapter exactly zero in their windows."""
    check_rows(c, got, ref, what)
    inside = windows(c)
    dg, dr = as_f64(got)[:, inside], ref[:, inside]
    rel = float(np.linalg.norm(dg - dr) / np.linalg.norm(dr))
    assert rel <= DELTA_L2[c.dtype], f"{what}: relative L2 of the delta {rel:.3e}"
    return rel


@pytest.mark.parametrize("k", [2, 3, 4, 5, 6])
def test_workload_store_mode_delta(L, k):
    c = W.config(k)
    print(f"[fullsize-store] {c.name} T={c.T}", flush=True)
    d = DevCase(c)
    y, _ = d.apply(L, mode="auto", add=False)
    rows = np.arange(c.T) if c.T <= 256 else sample_rows(c)
    got = from_dev(y.index_select(0, torch.from_numpy(rows).cuda()))
    ref = oracle_rows(c, rows, add=False)
    rel = delta_gates(c, got, ref, c.name)
    none = rows[c.token_slot[rows] < 0]
    if none.size:
        z = as_f64(from_dev(y.index_select(0, torch.from_numpy(none).cuda())))[:, windows(c)]
        assert np.all(z == 0)
    print(f"[fullsize-store] {c.name}: {rows.shape[0]} rows, relative L2 of the delta {rel:.2e}", flush=True)
    del y, d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [7, 8])
def test_moe_workload_store_mode_delta(L, k):
    c = W.config(k)
    print(f"[fullsize-store] {c.name} pairs={c.rows}", flush=True)
    d = MoeDev(c)
    y, _ = d.apply(L, mode="auto", add=False)
    rng = np.random.Generator(np.random.PCG64(70 + k))
    rows = np.unique(np.concatenate([[0, c.rows - 1], rng.integers(0, c.rows, 160)])).astype(np.int64)
    got = from_dev(y.index_select(0, torch.from_numpy(rows).cuda()))
    ref = moe_ref(c, rows=rows, add=False)
    inside = windows(c)
    err = np.abs(as_f64(got) - ref)
    assert np.all(err <= 2e-2 * (1 + np.abs(ref))), c.name
    nz = np.linalg.norm(ref[:, inside])
    if nz > 0:
        rel = float(np.linalg.norm(as_f64(got)[:, inside] - ref[:, inside]) / nz)
        assert rel <= DELTA_L2["bf16"], f"{c.name}: relative L2 of the delta {rel:.3e}"
    del y, d
    torch.cuda.empty_cache()


def integer_like(c, seed):
    """The same batch (token slots, shapes, slices, per-slot rank padding) with
    sparse {-1, 0, 1} x, A, B and small-integer y0, so that every partial sum
    is a small integer: exact in fp32, and |u|, |y| <= 256 keeps them exact in
    bf16.  The bound is checked on the oracle's result."""
    rng = np.random.Generator(np.random.PCG64(seed))

    def sparse(shape, p):
        v = np.zeros(shape, np.float32)
        m = rng.random(shape, dtype=np.float32) < p
        v[m] = rng.choice(np.array([-1.0, 1.0], np.float32), int(m.sum()))
        return W.bf16_round(v)

    c.x = sparse(c.x.shape, 0.25)
    ranks = np.asarray(c.ranks)
    A, B = [], []
    for a, b in zip(c.A, c.B):
        a = sparse(a.shape, 32.0 / c.d_in)
        b = sparse(b.shape, 3.0 / c.r_max)
        for s in range(c.num_slots):      # keep each slot's zero padding past its rank
            a[s, :, ranks[s]:] = 0
            b[s, ranks[s]:, :] = 0
        A.append(a)
        B.append(b)
    c.A, c.B = A, B
    y0 = rng.integers(-8, 9, c.y0.shape, dtype=np.int8)
    c.y0 = W.bf16_round(y0.astype(np.float32))
    return c


@pytest.mark.parametrize("k", [5, 3])
def test_integer_inputs_bit_exact_at_workload_plans(L, k):
    """Integer inputs on the exact batch plan of workload 5 (the tile kernels'
    short-tile plan with d_in split into k-chunks) and of workload 3 (the
    long-segment expand over 17 705 tokens): every sampled row bit-identical to
    the oracle, in the launch configuration the benchmark times (AUTO, add)."""
    c = integer_like(W.config(k), 900 + k)
    print(f"[fullsize-int] {c.name} T={c.T}", flush=True)
    rows = sample_rows(c, k_random=64, seed=k)
    ref, u = oracle_rows(c, rows, return_u=True)
    assert np.max(np.abs(u)) <= 256 and np.max(np.abs(ref)) <= 256
    assert np.all(ref == np.round(ref))
    d = DevCase(c)
    y, _ = d.apply(L, mode="auto", add=True)
    got = as_f64(from_dev(y.index_select(0, torch.from_numpy(rows).cuda())))
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{c.name}: {bad.shape[0]} elements differ, first at row {rows[bad[0][0]]} col {bad[0][1]}"
    print(f"[fullsize-int] {c.name}: {rows.shape[0]} rows bit-exact", flush=True)
    del y, d
    torch.cuda.empty_cache()
