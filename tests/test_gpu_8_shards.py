"""One GPU's share of a sharded layer.  The plans for more than one GPU
(tensor-parallel column shards of B, row shards of d_in, rank shards of A and
B with an all-gather of the rank-r buffer; page "vLLM 源码完全拆解(十八):多 LoRA
服务", section "张量并行下的 LoRA") are computed here shard by shard on one GPU
with the library's entry points, and combined on the device the way the
collective would combine them; the result must be the oracle's unsharded
layer."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, DevCase, as_f64, check_rows, from_dev, oracle_rows, to_dev
from test_gpu_2_apply import small_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["auto", "sgmv"])
def test_column_shards(L, dtype, mode):
    """Column-parallel layer: shard j holds columns [c0, c1) of every slice of
    B and writes only them; together the shards write every window, with no
    exchange."""
    c = small_case(900, dtype, 32)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    for j in range(2):
        Bj, offs = [], []
        for b, w, o in zip(c.B, c.widths, c.offsets):
            c0, c1 = (w // 2 // 8 * 8, w) if j else (0, w // 2 // 8 * 8)
            Bj.append(to_dev(np.ascontiguousarray(b[:, :, c0:c1]), dtype))
            offs.append(o + c0)
        L.lora_apply(meta, d.x, d.A, Bj, offs, y, scale=c.scale, slot_scale=d.slot_scale, mode=mode)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), f"{c.name} column shards")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["auto", "sgmv"])
def test_row_shards(L, dtype, mode):
    """Row-parallel layer: shard j holds rows [k0, k1) of d_in (its part of x
    and of A) and produces a partial delta; the sum of the partial deltas (the
    base layer's all-reduce) plus the base output is the layer's output."""
    c = small_case(910, dtype, 32)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    k_split = 128
    total = torch.zeros_like(d.y0, dtype=torch.float32)
    for k0, k1 in ((0, k_split), (k_split, c.d_in)):
        xj = d.x[:, k0:k1]                       # a strided view: row stride d_in
        Aj = [to_dev(np.ascontiguousarray(a[:, k0:k1, :]), dtype) for a in c.A]
        part = torch.zeros_like(d.y0)
        L.lora_apply(meta, xj, Aj, d.B, c.offsets, part, scale=c.scale, slot_scale=d.slot_scale, add=False,
                     mode=mode)
        total += part.float()
    got = (d.y0.float() + total).cpu().numpy().astype(np.float64)
    ref = oracle_rows(c, np.arange(c.T))
    # each partial delta was rounded once when stored: twice the one-store bound
    tol = 2 * TOL[c.dtype]
    bad = np.abs(got - ref) > tol * (1.0 + np.abs(ref))
    assert not bad.any(), f"{int(bad.sum())} elements out of tolerance"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rank_shards_gather_u(L, dtype):
    """Rank shards (S-LoRA style): shard j holds ranks [r0, r1) of A; each
    shrinks into its own slice of the rank-r buffer, the slices are gathered
    along the rank dimension (the all-gather), and the expand with the whole B
    gives the layer's output."""
    c = small_case(920, dtype, 64)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    us = []
    for r0, r1 in ((0, 32), (32, 64)):
        Aj = [to_dev(np.ascontiguousarray(a[:, :, r0:r1]), dtype) for a in c.A]
        uj = torch.zeros((c.n_slices, c.T, r1 - r0), dtype=torch.float32, device="cuda")
        L.lora_shrink(meta, d.x, Aj, uj, scale=c.scale, slot_scale=d.slot_scale, mode="sgmv")
        us.append(uj)
    u = torch.cat(us, dim=2).contiguous()
    y = d.y0.clone()
    L.lora_expand(meta, u, d.B, c.offsets, y, add=True, mode="sgmv")
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), f"{c.name} rank shards")
