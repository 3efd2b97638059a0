"""B in the output-rows layout (LORA_LAYOUT_OUT_ROWS): B_s[slot] as
[w][r_max], one row of ranks per output column, the stacked B of page
"vLLM 源码完全拆解(十八):多 LoRA 服务", section "包装层的形态".  The oracle
keeps the default [r][w] B and the device gets the transposed copy, so both
see the same factors.  Cases: the small mixed batch at every rank the tile
expand takes (r_max on and off the tile ranks), both A layouts, per-slot ranks
with NaN past them, add and store, the expand alone from a seeded rank-r
buffer, long segments and decode batches (which lora_apply then runs on the
tile kernels), integer inputs that every summation order gets exactly, and the
prefill and many-adapter decode workloads at full size."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DELTA_L2, DevCase, as_f64, check_rows, from_dev, oracle_rows, sample_rows, to_dev
from test_gpu_10_fullsize import delta_gates
from test_gpu_2_apply import small_case
from test_gpu_4_edges import integer_case
from test_gpu_6_ranks import nan_padded, rank_rows
from test_gpu_11_long_segments import long_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def out_rows(B_list, dtype):
    """[S][r][w] -> [S][w][r] on the device."""
    return [to_dev(np.ascontiguousarray(np.transpose(b, (0, 2, 1))), dtype) for b in B_list]


def apply_out(L, c, d, B, mode="auto", add=True, ranks=None, A=None, a_rank_rows=False):
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    L.lora_apply(meta, d.x, d.A if A is None else A, B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale,
                 add=add, mode=mode, slot_rank=ranks, a_rank_rows=a_rank_rows, b_out_rows=True)
    return from_dev(y)


@pytest.mark.parametrize("r", [8, 16, 24, 32, 48, 64])
@pytest.mark.parametrize("mode", ["auto", "sgmv"])
def test_b_out_rows_apply_small(L, r, mode):
    c = small_case(1500 + r, "bf16", r)
    print(f"[b-out] {c.name} mode={mode}", flush=True)
    d = DevCase(c)
    B = out_rows(c.B, c.dtype)
    for add in (True, False):
        got = apply_out(L, c, d, B, mode=mode, add=add)
        ref = oracle_rows(c, np.arange(c.T), add=add)
        check_rows(c, got, ref, f"{c.name} add={add}")
        if not add:
            err = np.linalg.norm(as_f64(got) - ref) / max(np.linalg.norm(ref), 1e-30)
            assert err <= DELTA_L2["bf16"], err


@pytest.mark.parametrize("r", [16, 32, 64])
@pytest.mark.parametrize("a_rank_rows", [False, True])
def test_b_out_rows_slot_ranks(L, r, a_rank_rows):
    """NaN past each slot's rank (rounded up to 8) in both factors: a read of
    the padding would turn rows into NaN."""
    c = small_case(1600 + r, "bf16", r)
    d = DevCase(c)
    A_nan, B_nan = nan_padded(c)
    A = rank_rows(A_nan, c.dtype) if a_rank_rows else [to_dev(a, c.dtype) for a in A_nan]
    ranks = torch.from_numpy(np.asarray(c.ranks, np.int32)).cuda()
    for add in (True, False):
        got = apply_out(L, c, d, out_rows(B_nan, c.dtype), add=add, ranks=ranks, A=A, a_rank_rows=a_rank_rows)
        check_rows(c, got, oracle_rows(c, np.arange(c.T), add=add), f"{c.name} add={add}")


@pytest.mark.parametrize("r", [8, 16, 32, 64])
@pytest.mark.parametrize("add", [True, False])
def test_b_out_rows_expand_alone(L, r, add):
    """lora_expand from a seeded fp32 rank-r buffer (drawn by the input
    generator, so neither side consumes a result of the other)."""
    c = small_case(1700 + r, "bf16", r)
    rng = np.random.Generator(np.random.PCG64(17 + r))
    u_np = rng.standard_normal((c.n_slices, c.T, r), dtype=np.float32)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    L.lora_expand(meta, torch.from_numpy(u_np).cuda(), out_rows(c.B, c.dtype), c.offsets, y, add=add,
                  b_out_rows=True)
    ref = oracle.expand_rows(u_np, c.token_slot, c.num_slots, c.B, c.offsets, c.y0, add=add)
    check_rows(c, from_dev(y), ref, f"{c.name} add={add}")


@pytest.mark.parametrize("shape", ["decode_q4096_r16", "prefill_gateup_r64", "qkv_r32"])
def test_b_out_rows_integer_bit_exact(L, shape):
    if shape == "decode_q4096_r16":
        c = integer_case(1811, [1] * 256, 32, 4096, [4096], 16, 2.0)
    elif shape == "prefill_gateup_r64":
        c = integer_case(1812, [300, 1, 700, 64, 129], 8, 4096, [2048, 2048], 64, 1.0)
    else:
        c = integer_case(1813, [1] * 200 + [513, 257], 64, 4096, [4096, 1024, 1024], 32, 2.0)
    print(f"[b-out-int] {shape} T={c.T}", flush=True)
    ref = oracle_rows(c, np.arange(c.T))
    assert np.max(np.abs(ref)) <= 256 and np.all(ref == np.round(ref))
    d = DevCase(c)
    B = out_rows(c.B, c.dtype)
    for mode in ("auto", "sgmv"):
        assert np.array_equal(as_f64(apply_out(L, c, d, B, mode=mode)), ref), mode


@pytest.mark.parametrize("r,d_in,widths", [(64, 1024, [384, 256]), (32, 2056, [512, 128, 128]), (24, 1536, [264])])
def test_b_out_rows_long_segments(L, r, d_in, widths):
    """Segments of hundreds of tokens: lora_apply takes the tile expand for
    this layout where the default one would take the long-segment expand."""
    c = long_case(1900 + r, r, d_in, widths)
    d = DevCase(c)
    B = out_rows(c.B, c.dtype)
    for add in (True, False):
        check_rows(c, apply_out(L, c, d, B, add=add), oracle_rows(c, np.arange(c.T), add=add), f"{c.name} add={add}")


def test_b_out_rows_matches_default_layout_on_decode(L):
    """A decode batch (one token per request): the default layout runs the
    split decode kernel, this one the tile kernels; both match the oracle."""
    rng = np.random.Generator(np.random.PCG64(2000))
    req = rng.integers(-1, 32, 256).astype(np.int32)
    c = W.make_case(name="b_out_decode", seed=2000, rng=rng, dtype="bf16", lengths=np.ones(256, np.int64),
                    req_slot=req, num_slots=32, d_in=4096, r_max=16, widths=[4096], weight_sd=0.05)
    d = DevCase(c)
    ref = oracle_rows(c, np.arange(c.T))
    check_rows(c, apply_out(L, c, d, out_rows(c.B, c.dtype)), ref, "out rows")
    y, _ = d.apply(L)
    check_rows(c, from_dev(y), ref, "default layout")


def test_b_out_rows_rejected_calls(L):
    """fp32 and mode BGMV are not served in this layout (r_max 128 neither:
    the argument checks run on the CPU too)."""
    c = small_case(2100, "f32", 16)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    with pytest.raises(L.LoraError) as e:
        L.lora_apply(meta, d.x, d.A, out_rows(c.B, c.dtype), c.offsets, d.y0.clone(), b_out_rows=True)
    assert e.value.status == L.LORA_ERR_UNSUPPORTED
    c = small_case(2101, "bf16", 16)
    d = DevCase(c)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    with pytest.raises(L.LoraError) as e:
        L.lora_apply(meta, d.x, d.A, out_rows(c.B, c.dtype), c.offsets, d.y0.clone(), mode="bgmv", b_out_rows=True)
    assert e.value.status == L.LORA_ERR_UNSUPPORTED


@pytest.mark.parametrize("k", [3, 5])
def test_b_out_rows_full_size_store_mode(L, k):
    """The prefill gate/up and many-adapter decode workloads at full size with
    output-major B, in store mode (the gates then apply to the delta itself),
    on the sampled rows."""
    c = W.config(k)
    print(f"[b-out-full] {c.name} T={c.T}", flush=True)
    d = DevCase(c)
    B = out_rows(c.B, c.dtype)
    meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
    y = d.y0.clone()
    L.lora_apply(meta, d.x, d.A, B, c.offsets, y, scale=c.scale, add=False, b_out_rows=True)
    rows = sample_rows(c)
    got = from_dev(y.index_select(0, torch.from_numpy(rows).cuda()))
    delta_gates(c, got, oracle_rows(c, rows, add=False), f"{c.name} b_out_rows")
    del y, d, B
    torch.cuda.empty_cache()
