"""Edge cases on the GPU: empty and all-none batches, invalid slot ids,
integer-valued inputs that every summation order gets exactly (so the GPU must
match the oracle bit for bit at real shapes), workspace reuse, and 64-bit row
offsets (T * ldy above 2^31)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import DevCase, as_f64, check_rows, from_dev, oracle_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def test_empty_batch(L):
    """T = 0: metadata says no adapter, apply is a successful no-op."""
    ts = torch.zeros(0, dtype=torch.int32, device="cuda")
    meta = L.lora_prepare_meta(ts, 4)
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(4, 64, 16, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(4, 16, 64, dtype=torch.bfloat16, device="cuda")
    L.lora_apply(meta, x, [A], [B], [0], y, scale=1.0)
    torch.cuda.synchronize()
    info = meta.tensors()["info"].cpu().numpy()
    assert info[0] == 0 and info[1] == 1


@pytest.mark.parametrize("add", [True, False])
def test_all_none(L, add):
    rng = np.random.Generator(np.random.PCG64(3))
    c = W.make_case(name="none", seed=3, rng=rng, dtype="bf16", lengths=np.ones(300, np.int64),
                    req_slot=np.full(300, -1, np.int32), num_slots=4, d_in=128, r_max=16,
                    widths=[256], offsets=[64], ldy=384)
    d = DevCase(c)
    y, meta = d.apply(L, add=add)
    got = from_dev(y)
    if add:
        assert np.array_equal(got, c.y0)
    else:
        assert np.all(got[:, 64:320] == 0) and np.array_equal(got[:, :64], c.y0[:, :64])
        assert np.array_equal(got[:, 320:], c.y0[:, 320:])


def test_invalid_slot_ids_are_none(L):
    rng = np.random.Generator(np.random.PCG64(4))
    ts = rng.integers(-4, 10, 500).astype(np.int32)      # S = 6: ids < -1 or >= 6 are bad
    c = W.make_case(name="bad", seed=4, rng=rng, dtype="bf16", lengths=np.ones(500, np.int64),
                    req_slot=np.zeros(500, np.int32), num_slots=6, d_in=64, r_max=16, widths=[64],
                    token_slot=ts)
    d = DevCase(c)
    y, meta = d.apply(L)
    info = meta.tensors()["info"].cpu().numpy()
    assert info[2] == int(np.sum((ts < -1) | (ts >= 6)))
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), "bad ids")


def integer_case(seed, T_lengths, S, d_in, widths, r, scale, dtype="bf16", ldy=None, offsets=None):
    """Sparse {-1,0,1} x, A, B and small-integer y0: every partial sum is a
    small integer, exact in fp32, and |u|, |y| <= 256 keeps them exact in bf16
    too.  The constraint is checked on the oracle's result."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(T_lengths, np.int64)
    req = rng.integers(-1, S, lengths.shape[0]).astype(np.int32)
    c = W.make_case(name=f"int_{seed}", seed=seed, rng=rng, dtype=dtype, lengths=lengths, req_slot=req,
                    num_slots=S, d_in=d_in, r_max=r, widths=widths, offsets=offsets, ldy=ldy,
                    scale=scale)

    def sparse(shape, p):
        v = rng.choice(np.array([-1.0, 1.0], np.float32), shape) * (rng.random(shape) < p)
        return v.astype(np.float32)
    conv = W.bf16_round if dtype == "bf16" else (lambda a: a.astype(np.float32))
    c.x = conv(sparse(c.x.shape, 0.25))
    c.A = [conv(sparse(a.shape, 32.0 / d_in)) for a in c.A]
    c.B = [conv(sparse(b.shape, 3.0 / r)) for b in c.B]
    c.y0 = conv(rng.integers(-8, 9, c.y0.shape).astype(np.float32))
    return c


@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
@pytest.mark.parametrize("shape", ["decode_q4096_r16", "prefill_gateup_r64", "qkv_r32"])
def test_integer_inputs_bit_exact(L, mode, shape):
    if shape == "decode_q4096_r16":
        c = integer_case(11, [1] * 256, 32, 4096, [4096], 16, 2.0)
    elif shape == "prefill_gateup_r64":
        c = integer_case(12, [300, 1, 700, 64, 129], 8, 4096, [2048, 2048], 64, 1.0)
    else:
        c = integer_case(13, [1] * 200 + [513, 257], 64, 4096, [4096, 1024, 1024], 32, 2.0,
                         offsets=[0, 4096, 5120], ldy=6144)
    print(f"[int] {shape} mode={mode} T={c.T}", flush=True)
    ref, u = oracle_rows(c, np.arange(c.T), return_u=True)
    assert np.max(np.abs(u)) <= 256 and np.max(np.abs(ref)) <= 256
    assert np.all(ref == np.round(ref))
    d = DevCase(c)
    y, _ = d.apply(L, mode=mode)
    assert np.array_equal(as_f64(from_dev(y)), ref)


def test_workspace_reuse_two_shapes(L):
    """One apply workspace serves calls of different sizes in a row: garbage
    everywhere except the count words, which lora_apply_workspace_init
    clears once."""
    from test_gpu_2_apply import small_case
    big = W.config(5)
    dbig = DevCase(big)
    small = small_case(77, "bf16", 64)
    dsmall = DevCase(small)
    need = max(L.lora_apply_workspace_bytes(big.T, big.num_slots, big.d_in, 1, 64, torch.bfloat16),
               L.lora_apply_workspace_bytes(small.T, small.num_slots, small.d_in, 3, 64, torch.bfloat16))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    L.lora_apply_workspace_init(ws)
    rows = np.arange(0, big.T, 97)
    for _ in range(2):
        yb, _ = dbig.apply(L, workspace=ws)
        ys, _ = dsmall.apply(L, workspace=ws)
        check_rows(big, from_dev(yb.index_select(0, torch.from_numpy(rows).cuda())),
                   oracle_rows(big, rows), "big")
        check_rows(small, from_dev(ys), oracle_rows(small, np.arange(small.T)), "small")


def test_int64_row_offsets(L):
    """T * ldy > 2^31 elements: rows past 2^31 / ldy are addressed correctly."""
    T, ldy, d_in, r, S = 70000, 32768, 64, 16, 4
    rng = np.random.Generator(np.random.PCG64(21))
    ts = rng.integers(-1, S, T).astype(np.int32)
    x = W.bf16_round(rng.standard_normal((T, d_in), dtype=np.float32))
    A = W.bf16_round(0.1 * rng.standard_normal((S, d_in, r), dtype=np.float32))
    B = W.bf16_round(0.1 * rng.standard_normal((S, r, ldy), dtype=np.float32))
    assert T * ldy > 2 ** 31
    y = torch.zeros(T, ldy, dtype=torch.bfloat16, device="cuda")
    meta = L.lora_prepare_meta(torch.from_numpy(ts).cuda(), S)
    L.lora_apply(meta, to_dev(x, "bf16"), [to_dev(A, "bf16")], [to_dev(B, "bf16")], [0], y, scale=1.0)
    rows = np.array([0, 1, 65535, 65536, 65537, 69998, 69999] + list(rng.integers(65536, T, 8)), np.int64)
    got = from_dev(y.index_select(0, torch.from_numpy(rows).cuda()))
    ref = oracle.lora_rows(x[rows], ts[rows], S, [A], [B], [0], 1.0,
                           np.zeros((rows.shape[0], ldy), np.uint16))
    assert np.all(np.abs(as_f64(got) - ref) <= 2e-2 * (1 + np.abs(ref)))
    del y
    torch.cuda.empty_cache()
