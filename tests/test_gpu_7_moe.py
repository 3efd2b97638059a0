"""The experts' LoRA of a top-k MoE layer: pairs (token, choice) keyed by
(slot, local expert).  Metadata bit-exact against the oracle's keys run through
the oracle's metadata; the gate/up LoRA (x row = pair / topk) and the down LoRA
(x row = pair) against the oracle's fp64 rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import TOL, as_f64, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def small_moe(seed, dtype="bf16", per_pair=False, T=75, K=4, S=3, E=24, EL=6, r=16, widths=(40, 72),
              with_map=True, bad=False):
    """A small MoE step that spans several 64-row tiles and a ragged tail:
    experts of this rank are a scattered subset of the global ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ts = rng.integers(-1, S, T).astype(np.int32)
    emap = None
    if with_map:
        emap = np.full(E, -1, np.int32)
        emap[rng.permutation(E)[:EL]] = np.arange(EL, dtype=np.int32)
    if bad:
        ts[3] = S + 2
        topk[5, 1] = E + 7
        if emap is not None:
            emap[int(topk[9, 0])] = EL + 1
    d_in = 96
    widths = list(widths)
    offsets = list(np.cumsum([0] + widths[:-1]))
    ldy = sum(widths) + 8
    x = W._draw(rng, ((T * K) if per_pair else T, d_in), 1.0, dtype)
    A = [W._draw(rng, (S, EL, d_in, r), 0.1, dtype) for _ in widths]
    B = [W._draw(rng, (S, EL, r, w), 0.1, dtype) for w in widths]
    y0 = W._draw(rng, (T * K, ldy), 1.0, dtype)
    return W.MoeCase(name=f"moe_small_{seed}", dtype=dtype, token_slot=ts, topk_ids=topk, expert_map=emap,
                     num_slots=S, num_experts=E, num_local_experts=EL, d_in=d_in, r_max=r,
                     ranks=np.full(S, r, np.int32), widths=widths, offsets=offsets, ldy=ldy, scale=0.5,
                     x=x, x_per_pair=per_pair, A=A, B=B, y0=y0, seed=seed)


class MoeDev:
    def __init__(self, c: W.MoeCase):
        self.c = c
        self.topk_ids = torch.from_numpy(c.topk_ids).cuda()
        self.token_slot = torch.from_numpy(c.token_slot).cuda()
        self.expert_map = None if c.expert_map is None else torch.from_numpy(c.expert_map).cuda()
        SE = c.num_slots * c.num_local_experts
        self.x = to_dev(c.x, c.dtype)
        self.A = [to_dev(a, c.dtype).view(SE, *a.shape[2:]) for a in c.A]
        self.B = [to_dev(b, c.dtype).view(SE, *b.shape[2:]) for b in c.B]
        self.y0 = to_dev(c.y0, c.dtype)

    def meta(self, L):
        c = self.c
        m = L.lora_prepare_moe_meta(self.topk_ids, self.token_slot, c.num_slots, c.num_experts,
                                    c.num_local_experts, self.expert_map)
        return m.with_x_row_div(1) if c.x_per_pair else m

    def apply(self, L, mode="auto", add=True):
        m = self.meta(L)
        y = self.y0.clone()
        L.lora_apply(m, self.x, self.A, self.B, self.c.offsets, y, scale=self.c.scale, add=add, mode=mode)
        return y, m


def moe_ref(c: W.MoeCase, rows=None, add=True):
    return oracle.moe_rows(c.x, c.topk_ids, c.token_slot, c.num_slots, c.num_experts, c.num_local_experts,
                           c.A, c.B, c.offsets, c.scale, c.y0, expert_map=c.expert_map,
                           x_per_pair=c.x_per_pair, add=add, rows=rows)


def check(c, got, ref, what):
    got = as_f64(got)
    tol = TOL[c.dtype]
    bad = np.abs(got - ref) > tol * (1.0 + np.abs(ref))
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} out of tolerance; first ({i},{j}) "
                             f"got {got[i, j]!r} ref {ref[i, j]!r}")


def check_meta(L, d: MoeDev):
    c = d.c
    keys = oracle.moe_keys(c.topk_ids, c.token_slot, c.num_slots, c.num_experts, c.num_local_experts,
                           c.expert_map)
    ref = oracle.prepare_meta(keys, c.num_slots * c.num_local_experts)
    m = d.meta(L)
    torch.cuda.synchronize()
    assert m.num_tokens == c.rows and m.num_slots == c.num_slots * c.num_local_experts
    assert int(m.c.x_row_div) == (1 if c.x_per_pair else c.topk)
    t = {k: v.cpu().numpy() for k, v in m.tensors().items()}
    np.testing.assert_array_equal(t["sorted"], ref.sorted)
    np.testing.assert_array_equal(t["seg_slot"], ref.seg_slot)
    np.testing.assert_array_equal(t["seg_count"], ref.seg_count)
    np.testing.assert_array_equal(t["seg_start"], ref.seg_start)
    assert t["info"][0] == ref.num_segments and t["info"][1] == ref.no_lora and t["info"][2] == ref.num_bad
    return ref


@pytest.mark.parametrize("seed,with_map,bad", [(1, True, False), (2, False, False), (3, True, True),
                                               (4, False, True)])
def test_moe_meta_bit_exact(L, seed, with_map, bad):
    c = small_moe(700 + seed, with_map=with_map, bad=bad, EL=6 if with_map else 24)
    print(f"[moe-meta] {c.name} map={with_map} bad={bad}", flush=True)
    ref = check_meta(L, MoeDev(c))
    assert (ref.num_bad > 0) == bad


@pytest.mark.parametrize("with_map,bad", [(True, False), (False, True)])
def test_moe_meta_many_rows(L, with_map, bad):
    """1100 tokens x top-8: 8800 (token, expert) rows, counted in parts by
    several workgroups; the apply on them too."""
    c = small_moe(740 + int(bad), T=1100, K=8, E=64, EL=16 if with_map else 64, with_map=with_map, bad=bad)
    print(f"[moe-meta] {c.name} rows={c.rows} map={with_map} bad={bad}", flush=True)
    d = MoeDev(c)
    ref = check_meta(L, d)
    assert (ref.num_bad > 0) == bad
    y, _ = d.apply(L)
    rows = np.arange(0, c.rows, 7)
    check(c, from_dev(y)[rows], moe_ref(c, rows=rows), c.name)


@pytest.mark.parametrize("with_map,bad", [(True, False), (False, True)])
def test_moe_meta_one_workgroup_scattered(L, with_map, bad):
    """600 tokens x top-8: 4800 (token, expert) rows of many keys in batch
    order, on one workgroup, whose scatter then goes through LDS."""
    c = small_moe(760 + int(bad), T=600, K=8, E=64, EL=16 if with_map else 64, with_map=with_map, bad=bad)
    print(f"[moe-meta] {c.name} rows={c.rows} map={with_map} bad={bad}", flush=True)
    d = MoeDev(c)
    ref = check_meta(L, d)
    assert (ref.num_bad > 0) == bad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("per_pair", [False, True])
@pytest.mark.parametrize("mode", ["auto", "bgmv", "sgmv"])
def test_moe_apply_small(L, dtype, per_pair, mode):
    c = small_moe(720, dtype=dtype, per_pair=per_pair)
    print(f"[moe-apply] {c.name} {dtype} per_pair={per_pair} mode={mode}", flush=True)
    d = MoeDev(c)
    for add in (True, False):
        y, _ = d.apply(L, mode=mode, add=add)
        check(c, from_dev(y), moe_ref(c, add=add), f"{c.name} add={add}")


def test_moe_shrink_expand_split(L):
    """Shrink and expand called one after the other on MoE metadata: u holds a
    row per pair, and the expand adds the pairs' deltas."""
    c = small_moe(730, dtype="bf16")
    d = MoeDev(c)
    m = d.meta(L)
    u = torch.zeros((len(c.A), c.rows, c.r_max), dtype=torch.float32, device="cuda")
    L.lora_shrink(m, d.x, d.A, u, scale=c.scale, mode="sgmv")
    y = d.y0.clone()
    L.lora_expand(m, u, d.B, c.offsets, y, add=True, mode="sgmv")
    check(c, from_dev(y), moe_ref(c), c.name)


def test_moe_integer_bit_exact(L):
    """Small-integer factors: every product and sum is exact in fp32, so the
    result is bit-exact against the oracle."""
    c = small_moe(740, dtype="f32", per_pair=False, r=8)
    rng = np.random.Generator(np.random.PCG64(741))
    c.x = rng.integers(-3, 4, c.x.shape).astype(np.float32)
    c.A = [rng.integers(-2, 3, a.shape).astype(np.float32) for a in c.A]
    c.B = [rng.integers(-2, 3, b.shape).astype(np.float32) for b in c.B]
    c.y0 = rng.integers(-50, 51, c.y0.shape).astype(np.float32)
    c.scale = 1.0
    d = MoeDev(c)
    for mode in ("bgmv", "sgmv"):
        y, _ = d.apply(L, mode=mode)
        np.testing.assert_array_equal(from_dev(y).astype(np.float64), moe_ref(c))


def test_moe_no_local_expert(L):
    """An expert map with no local expert among the choices leaves y as it was."""
    c = small_moe(750, dtype="bf16")
    c.expert_map = np.full(c.num_experts, -1, np.int32)
    d = MoeDev(c)
    y, m = d.apply(L)
    torch.cuda.synchronize()
    assert int(m.tensors()["info"][1].item()) == 1
    assert torch.equal(y, d.y0)


@pytest.mark.parametrize("k", [7, 8])
def test_moe_workload_parity(L, k):
    c = W.config(k)
    print(f"[moe-workload] {c.name} rows={c.rows}", flush=True)
    d = MoeDev(c)
    check_meta(L, d)
    y, _ = d.apply(L, mode="auto")
    rng = np.random.Generator(np.random.PCG64(k))
    rows = np.unique(np.concatenate([[0, c.rows - 1], rng.integers(0, c.rows, 96)])).astype(np.int64)
    got = from_dev(y.index_select(0, torch.from_numpy(rows).cuda()))
    check(c, got, moe_ref(c, rows=rows), c.name)
    # pairs whose expert is not on this rank, or whose token has no adapter, are untouched
    keys = oracle.moe_keys(c.topk_ids, c.token_slot, c.num_slots, c.num_experts, c.num_local_experts,
                           c.expert_map)
    none = torch.from_numpy(np.where(keys < 0)[0]).cuda()
    assert torch.equal(y.index_select(0, none), d.y0.index_select(0, none))
    del y, d
    torch.cuda.empty_cache()
