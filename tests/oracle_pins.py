"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, none of which goes through the oracle's own arithmetic.

Each ``pin_*`` takes a loaded oracle library and raises AssertionError when the
oracle disagrees.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake and requires that some pin catches each mistake.

Kinds of pin used here:
  * worked examples printed on the pages (tests/golden/*.json, each citing its
    passage);
  * brute force over every slot assignment of tiny batches against Python's
    stable ``sorted``;
  * closed forms evaluated with numpy matmul (different association order and
    summation code): the merged weight W + s*A*B of the handbook page, identity
    factors, per-slice block products;
  * exact invariants: scale linearity, slot relabelling, token permutation,
    rows without an adapter, zero-padded ranks, zero adapters.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _delta_np(x, A, B, slot, scale, slot_scale=None):
    """numpy closed form of one token-block's delta for one slice: s*(x@A)@B."""
    sc = scale * (1.0 if slot_scale is None else float(slot_scale[slot]))
    return sc * ((x.astype(np.float64) @ A[slot].astype(np.float64))
                 @ B[slot].astype(np.float64))


def _small_case(seed, T=23, S=5, d_in=40, r=8, widths=(24, 16), offsets=None,
                ldy=None, dtype="f32", no_lora_frac=0.2, ranks=None):
    rng = _rng(seed)
    lengths = np.ones(T, np.int64)
    req = rng.integers(0, S, T).astype(np.int32)
    return W.make_case(name="pin", seed=seed, rng=rng, dtype=dtype,
                       lengths=lengths, req_slot=req, num_slots=S, d_in=d_in,
                       r_max=r, widths=list(widths), offsets=offsets, ldy=ldy,
                       scale=1.5, no_lora_frac=no_lora_frac, weight_sd=0.3,
                       ranks=ranks)


def _rows(c, lib, add=True, **kw):
    return oracle.lora_rows(c.x, c.token_slot, c.num_slots, c.A, c.B, c.offsets,
                            c.scale, c.y0, add=add, lib=lib, **kw)


# --------------------------------------------------------------------------- metadata


def pin_meta_walkthrough(lib):
    g = _golden("meta_walkthrough.json")
    m = oracle.prepare_meta(np.array(g["token_slot"]), g["num_slots"], lib=lib)
    n = g["num_segments"]
    assert m.num_segments == n
    assert m.sorted.tolist() == g["sorted"]
    assert m.seg_slot[:n].tolist() == g["seg_slot"]
    assert m.seg_count[:n].tolist() == g["seg_count"]
    assert m.seg_start[:n + 1].tolist() == g["seg_start"]
    assert m.no_lora == g["no_lora"]


def pin_meta_running_example(lib):
    g = _golden("meta_running_example.json")
    ts = np.concatenate([np.full(v, int(k), np.int32) for k, v in g["counts_by_key"].items()])
    ts = ts[_rng(7).permutation(ts.shape[0])]
    m = oracle.prepare_meta(ts, g["num_slots"], lib=lib)
    n = len(g["seg_count"])
    assert m.seg_count[:n].tolist() == g["seg_count"]
    assert m.seg_start[:n + 1].tolist() == g["seg_start"]


def pin_meta_toy_segments(lib):
    g = _golden("handbook_toy_summary.json")["printed"]
    c = W.config(1)
    assert c.T == g["base_matmul_rows"] and len(c.lengths) == g["per_request_calls"]
    m = oracle.prepare_meta(c.token_slot, c.num_slots, lib=lib)
    assert m.num_segments == g["sgmv_segments"]


def _meta_reference(ts, S):
    """Python's stable sorted() plus counting, with out-of-range ids as -1."""
    eff = [v if -1 <= v < S else -1 for v in ts]
    order = sorted(range(len(eff)), key=lambda t: eff[t])
    keys = sorted(set(eff))
    counts = [eff.count(k) for k in keys]
    return order, keys, counts


def _check_meta(m, ts, S):
    order, keys, counts = _meta_reference(list(ts), S)
    T, n = len(ts), len(keys)
    assert m.sorted.tolist() == order
    assert m.num_segments == n
    assert m.seg_slot.tolist() == keys + [-1] * (S + 1 - n)
    assert m.seg_count.tolist() == counts + [0] * (S + 1 - n)
    assert m.seg_start.tolist() == list(np.cumsum([0] + counts)) + [T] * (S + 1 - n)
    assert m.no_lora == int(all(k == -1 for k in keys))


def pin_meta_bruteforce(lib):
    for S in (1, 2, 3):
        for T in range(0, 6 if S < 3 else 5):
            for ts in itertools.product(range(-1, S), repeat=T):
                ts = np.array(ts, np.int32)
                _check_meta(oracle.prepare_meta(ts, S, lib=lib), ts, S)


def pin_meta_invalid_and_large(lib):
    ts = np.array([3, -1, 7, -5, 0, 3, 99, 2, 2, -2], np.int32)   # S = 4: 7, -5, 99, -2 are bad
    m = oracle.prepare_meta(ts, 4, lib=lib)
    assert m.num_bad == 4
    _check_meta(m, [v if -1 <= v < 4 else -1 for v in ts.tolist()], 4)
    rng = _rng(11)
    for S, T in ((32, 2000), (128, 4096), (1, 300)):
        ts = rng.integers(-1, S, T).astype(np.int32)
        _check_meta(oracle.prepare_meta(ts, S, lib=lib), ts.tolist(), S)
    m = oracle.prepare_meta(np.full(17, -1, np.int32), 4, lib=lib)
    assert m.no_lora == 1 and m.num_segments == 1
    m = oracle.prepare_meta(np.zeros(0, np.int32), 4, lib=lib)
    assert m.no_lora == 1 and m.num_segments == 0 and m.seg_start.tolist() == [0] * 6


# --------------------------------------------------------------------------- y


def pin_handbook_toy_forms(lib):
    """The handbook's toy prints that its gathered (BGMV) and segmented (SGMV)
    forms both match the per-request loop to atol 1e-5.  Here the oracle's full
    output x*W + delta is checked against each of those three forms written with
    numpy (einsum over gathered factors; stable argsort + one matmul per
    segment; one matmul chain per request)."""
    g = _golden("handbook_toy_summary.json")["printed"]
    c = W.config(1)
    Wb = c.notes["W"].astype(np.float64)
    x = c.x.astype(np.float64)
    A, B = c.A[0].astype(np.float64), c.B[0].astype(np.float64)
    y0 = np.zeros((c.T, c.ldy), np.float32)
    y_or = oracle.lora_rows(c.x, c.token_slot, c.num_slots, c.A, c.B, [0],
                            c.scale, y0, add=True, lib=lib) + x @ Wb
    ts = c.token_slot
    gathered = np.einsum("tr,trn->tn", np.einsum("tk,tkr->tr", x, A[ts]), B[ts])
    bgmv = x @ Wb + c.scale * gathered
    order = np.argsort(ts, kind="stable")
    keys, counts = np.unique(ts[order], return_counts=True)
    assert len(keys) == g["sgmv_segments"]
    seg_out = np.empty((c.T, c.ldy))
    p = 0
    for k, n in zip(keys, counts):
        rows = order[p:p + n]
        seg_out[rows] = c.scale * (x[rows] @ A[k]) @ B[k]
        p += n
    sgmv = x @ Wb + seg_out
    per_req, p = [], 0
    for n, a in zip(c.lengths, c.req_slot):
        xi = x[p:p + n]
        per_req.append(xi @ Wb + c.scale * (xi @ A[a]) @ B[a])
        p += n
    per_req = np.concatenate(per_req)
    atol = g["allclose_atol"]
    for form in (bgmv, sgmv, per_req):
        assert np.allclose(y_or, form, atol=atol, rtol=0)
        assert np.max(np.abs(y_or - form)) <= 1e-10 * (1 + np.max(np.abs(form)))


def pin_merged_single_slot(lib):
    """Single-adapter batch: y = x (W + s A B) with the merged weight (handbook,
    the merged form is equivalent to the unmerged one); here W contributes y0."""
    c = _small_case(3, no_lora_frac=0.0, widths=(30,))
    c.token_slot[:] = 2
    y = _rows(c, lib)
    merged = c.scale * (c.A[0][2].astype(np.float64) @ c.B[0][2].astype(np.float64))
    ref = c.y0.astype(np.float64) + c.x.astype(np.float64) @ merged
    assert np.max(np.abs(y - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))


def pin_identity_factors(lib):
    """A = I (d_in = r): delta = s x B.  B = I (w = r): delta = s x A.  Small
    integers, so the results are exact."""
    rng = _rng(5)
    T, r, S = 9, 8, 3
    x = rng.integers(-3, 4, (T, r)).astype(np.float32)
    ts = np.array([0, 1, 2, 1, 0, 2, 2, 1, 0], np.int32)
    eye = np.stack([np.eye(r, dtype=np.float32)] * S)
    Bm = rng.integers(-2, 3, (S, r, 12)).astype(np.float32)
    y0 = rng.integers(-4, 5, (T, 12)).astype(np.float32)
    y = oracle.lora_rows(x, ts, S, [eye], [Bm], [0], 2.0, y0, lib=lib)
    ref = y0 + 2.0 * np.einsum("tk,tkn->tn", x.astype(np.float64), Bm[ts].astype(np.float64))
    assert np.array_equal(y, ref)
    Am = rng.integers(-2, 3, (S, 11, r)).astype(np.float32)
    x2 = rng.integers(-3, 4, (T, 11)).astype(np.float32)
    y0b = np.zeros((T, r), np.float32)
    y = oracle.lora_rows(x2, ts, S, [Am], [eye], [0], 3.0, y0b, lib=lib)
    ref = 3.0 * np.einsum("tk,tkr->tr", x2.astype(np.float64), Am[ts].astype(np.float64))
    assert np.array_equal(y, ref)


def pin_slices_blockwise(lib):
    """Unequal packed slices with a gap and a wider y: each window equals its own
    block product, columns outside every window stay y0."""
    c = _small_case(9, T=31, widths=(24, 8, 8), offsets=[0, 28, 40], ldy=52,
                    no_lora_frac=0.25)
    y = _rows(c, lib)
    ref = c.y0.astype(np.float64).copy()
    for t in range(c.T):
        a = c.token_slot[t]
        if a < 0:
            continue
        for s, (w, off) in enumerate(zip(c.widths, c.offsets)):
            ref[t, off:off + w] += _delta_np(c.x[t:t + 1], c.A[s], c.B[s], a, c.scale)[0]
    assert np.max(np.abs(y - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))
    outside = np.ones(c.ldy, bool)
    for w, off in zip(c.widths, c.offsets):
        outside[off:off + w] = False
    assert np.array_equal(y[:, outside], c.y0[:, outside].astype(np.float64))


def pin_add_flag_and_no_lora_rows(lib):
    c = _small_case(13, T=40, widths=(16, 16), offsets=[0, 20], ldy=40, no_lora_frac=0.3)
    none = c.token_slot == -1
    assert none.any()
    y_add = _rows(c, lib, add=True)
    y_set = _rows(c, lib, add=False)
    assert np.array_equal(y_add[none], c.y0[none].astype(np.float64))
    for w, off in zip(c.widths, c.offsets):
        assert np.all(y_set[none][:, off:off + w] == 0)
        # add == store + y0 in every window (fp64, |values| small: exact to ~1 ulp)
        d = y_add[:, off:off + w] - (y_set[:, off:off + w] + c.y0[:, off:off + w])
        assert np.max(np.abs(d)) <= 1e-13
    assert np.array_equal(y_set[:, 16:20], c.y0[:, 16:20].astype(np.float64))


def pin_scale_linearity_and_slot_scale(lib):
    """With the add flag clear the windows hold the delta itself (the windows
    cover every column here), so doubling s or a per-slot power-of-two scale
    must scale it exactly."""
    c = _small_case(17)
    d1 = _rows(c, lib, add=False)
    c2 = _small_case(17)
    c2.scale *= 2
    d2 = _rows(c2, lib, add=False)
    assert np.array_equal(d2, 2 * d1)
    ss = np.array([1.0, 0.5, 2.0, 4.0, 0.25], np.float32)
    d3 = _rows(c, lib, add=False, slot_scale=ss)
    mult = np.where(c.token_slot >= 0, ss[np.maximum(c.token_slot, 0)], 1.0)
    assert np.array_equal(d3, d1 * mult[:, None])


def pin_relabel_and_permute(lib):
    c = _small_case(19, T=29, S=6)
    y = _rows(c, lib)
    perm = _rng(1).permutation(c.num_slots)          # new slot id of old slot a is perm[a]
    inv = np.argsort(perm)
    c2 = _small_case(19, T=29, S=6)
    c2.token_slot = np.where(c.token_slot >= 0, perm[np.maximum(c.token_slot, 0)], -1).astype(np.int32)
    c2.A = [a[inv] for a in c.A]
    c2.B = [b[inv] for b in c.B]
    assert np.array_equal(_rows(c2, lib), y)
    tp = _rng(2).permutation(c.T)
    c3 = _small_case(19, T=29, S=6)
    c3.token_slot, c3.x, c3.y0 = c.token_slot[tp], c.x[tp], c.y0[tp]
    assert np.array_equal(_rows(c3, lib), y[tp])


def pin_zero_padding_and_zero_adapter(lib):
    ranks = np.array([8, 3, 5, 8, 1], np.int32)
    c = _small_case(23, ranks=ranks)
    y = _rows(c, lib)
    for a in range(c.num_slots):
        ra = int(ranks[a])
        sub = np.where(c.token_slot == a)[0]
        if sub.size == 0:
            continue
        A_t = [np.ascontiguousarray(x[:, :, :ra]) for x in c.A]
        B_t = [np.ascontiguousarray(b[:, :ra, :]) for b in c.B]
        y_t = oracle.lora_rows(c.x, c.token_slot, c.num_slots, A_t, B_t, c.offsets,
                               c.scale, c.y0, rows=sub, lib=lib)
        assert np.array_equal(y_t, y[sub])
    c.A = [np.zeros_like(a) for a in c.A]
    assert np.array_equal(_rows(c, lib), c.y0.astype(np.float64))


def pin_u_and_expand(lib):
    """The rank-r vectors equal s*x*A (numpy), and the expand alone from those
    vectors equals y0 + u*B."""
    c = _small_case(29, T=35, widths=(24, 16), dtype="bf16")
    y, u = _rows(c, lib, return_u=True)
    xf = W.to_f32(c.x).astype(np.float64)
    for s in range(c.n_slices):
        Af = W.to_f32(c.A[s]).astype(np.float64)
        for t in range(c.T):
            a = c.token_slot[t]
            ref = np.zeros(c.r_max) if a < 0 else c.scale * (xf[t] @ Af[a])
            assert np.max(np.abs(u[t, s] - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))
    u32 = np.ascontiguousarray(np.transpose(u, (1, 0, 2))).astype(np.float32)
    ye = oracle.expand_rows(u32, c.token_slot, c.num_slots, c.B, c.offsets, c.y0, lib=lib)
    ref = W.to_f32(c.y0).astype(np.float64).copy()
    for s, (w, off) in enumerate(zip(c.widths, c.offsets)):
        Bf = W.to_f32(c.B[s]).astype(np.float64)
        for t in range(c.T):
            a = c.token_slot[t]
            if a >= 0:
                ref[t, off:off + w] += u32[s, t].astype(np.float64) @ Bf[a]
    assert np.max(np.abs(ye - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))
    ye0 = oracle.expand_rows(u32, c.token_slot, c.num_slots, c.B, c.offsets, c.y0,
                             add=False, lib=lib)
    none = c.token_slot < 0
    assert np.all(ye0[none][:, :c.widths[0] + c.widths[1]] == 0)
    # same vectors give the same y through both entry points (to fp32 rounding of u)
    assert np.max(np.abs(ye - y)) <= 1e-5 * (1 + np.max(np.abs(y)))


def pin_bf16_inputs_exact(lib):
    """bf16 inputs are read as the exact values they encode: integer-valued
    bf16 data gives exactly the integer result."""
    rng = _rng(31)
    T, S, d, r, w = 12, 3, 64, 8, 24
    ints = lambda shape, lo, hi: rng.integers(lo, hi, shape).astype(np.float32)
    x, A, B, y0 = ints((T, d), -2, 3), ints((S, d, r), -1, 2), ints((S, r, w), -1, 2), ints((T, w), -8, 9)
    ts = rng.integers(-1, S, T).astype(np.int32)
    yb = oracle.lora_rows(W.bf16_round(x), ts, S, [W.bf16_round(A)], [W.bf16_round(B)], [0],
                          2.0, W.bf16_round(y0), lib=lib)
    yf = oracle.lora_rows(x, ts, S, [A], [B], [0], 2.0, y0, lib=lib)
    assert np.array_equal(yb, yf)
    ref = y0.astype(np.float64).copy()
    for t in range(T):
        if ts[t] >= 0:
            ref[t] += 2.0 * (x[t].astype(np.int64) @ A[ts[t]].astype(np.int64)
                             @ B[ts[t]].astype(np.int64))
    assert np.array_equal(yf, ref)


# --------------------------------------------------------------------------- MoE experts' LoRA

def _moe_case(seed, T=11, K=3, S=3, E_global=8, E_local=4, d_in=24, widths=(16, 8), r=8):
    """Tiny MoE step: top-K distinct experts per token, slots with -1, stacked
    per-(slot, local expert) factors [S][E_local][...]."""
    rng = _rng(seed)
    topk = np.stack([rng.permutation(E_global)[:K] for _ in range(T)]).astype(np.int32)
    ts = rng.integers(-1, S, T).astype(np.int32)
    x = rng.standard_normal((T, d_in)).astype(np.float32)
    A = [rng.standard_normal((S, E_local, d_in, r)).astype(np.float32) for _ in widths]
    B = [rng.standard_normal((S, E_local, r, w)).astype(np.float32) for w in widths]
    offsets = list(np.cumsum((0,) + tuple(widths))[:-1] + 4 * np.arange(len(widths)))
    ldy = int(offsets[-1] + widths[-1] + 4)
    y0 = rng.standard_normal((T * K, ldy)).astype(np.float32)
    return dict(x=x, topk=topk, ts=ts, S=S, E=E_global, EL=E_local, A=A, B=B, offsets=offsets, y0=y0)


def _moe(m, lib, expert_map=None, add=True, **kw):
    q = dict(m, **kw)
    return oracle.moe_rows(q["x"], q["topk"], q["ts"], q["S"], q["E"], q["EL"], q["A"], q["B"],
                           q["offsets"], 1.5, q["y0"], expert_map=expert_map, add=add, lib=lib)


def pin_moe_keys_by_hand(lib):
    """Keys worked out by hand from the definition: tokens on slots 1, -1, 0;
    experts 0..3 local (map to 0..3), 4..7 on another rank."""
    topk = np.array([[2, 5], [0, 1], [7, 3]], np.int32)
    emap = np.array([0, 1, 2, 3, -1, -1, -1, -1], np.int32)
    k = oracle.moe_keys(topk, np.array([1, -1, 0], np.int32), 2, 8, 4, emap, lib=lib)
    # t0: slot 1, expert 2 -> 1*4+2 = 6; expert 5 remote -> -1.  t1: no adapter.
    # t2: slot 0, expert 7 remote -> -1; expert 3 -> 0*4+3 = 3
    assert list(k) == [6, -1, -1, -1, -1, 3]
    # out of range: slot 5 >= S, expert 9 >= E, map entry 4 >= E_local; no map: expert 6 >= E_local
    k = oracle.moe_keys(np.array([[1], [9], [4]], np.int32), np.array([5, 0, 1], np.int32), 2, 8, 4,
                        np.array([0, 1, 2, 3, 4, -1, -1, -1], np.int32), lib=lib)
    assert list(k) == [-2, -2, -2]
    k = oracle.moe_keys(np.array([[6, 1]], np.int32), np.array([1], np.int32), 2, 8, 4, None, lib=lib)
    assert list(k) == [-2, 5]


def pin_moe_reduces_to_dense(lib):
    """One expert and top-1: the experts' LoRA is the dense LoRA of the tokens."""
    m = _moe_case(41, K=1, E_global=1, E_local=1)
    y = _moe(m, lib)
    yd = oracle.lora_rows(m["x"], m["ts"], m["S"], [a[:, 0] for a in m["A"]], [b[:, 0] for b in m["B"]],
                          m["offsets"], 1.5, m["y0"], lib=lib)
    assert np.array_equal(y, yd)


def pin_moe_pairs_closed_form(lib):
    """Every output row against numpy: row t*K + j adds 1.5 * x[t] @ A[a][e] @ B[a][e]
    on each slice window (or nothing), with e the local expert of the choice."""
    m = _moe_case(43)
    emap = np.array([3, -1, 0, 2, -1, 1, -1, -1], np.int32)
    y = _moe(m, lib, expert_map=emap)
    K = m["topk"].shape[1]
    ref = m["y0"].astype(np.float64).copy()
    for t in range(m["x"].shape[0]):
        a = int(m["ts"][t])
        for j in range(K):
            e = int(emap[m["topk"][t, j]])
            if a < 0 or e < 0:
                continue
            for s, o in enumerate(m["offsets"]):
                d = 1.5 * (m["x"][t].astype(np.float64) @ m["A"][s][a, e].astype(np.float64)) \
                    @ m["B"][s][a, e].astype(np.float64)
                ref[t * K + j, o:o + d.shape[0]] += d
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def pin_moe_expert_relabel(lib):
    """Renumbering the local experts together with their factor blocks and the
    expert map leaves every row unchanged."""
    m = _moe_case(47)
    emap = np.array([0, 1, 2, 3, -1, -1, -1, -1], np.int32)
    y = _moe(m, lib, expert_map=emap)
    sigma = np.array([2, 0, 3, 1])                     # old local id e -> new id sigma[e]
    inv = np.argsort(sigma)
    emap2 = np.where(emap >= 0, sigma[np.maximum(emap, 0)], -1).astype(np.int32)
    y2 = _moe(m, lib, expert_map=emap2, A=[a[:, inv] for a in m["A"]], B=[b[:, inv] for b in m["B"]])
    assert np.array_equal(y, y2)


def pin_moe_expert_parallel_partition(lib):
    """Two ranks holding experts 0..3 and 4..7: their deltas (stored, not
    added) sum to the delta of one rank holding all eight experts."""
    m = _moe_case(53, E_local=8)
    full = _moe(m, lib, add=False)
    parts = 0
    for rank in range(2):
        emap = np.array([e - 4 * rank if 4 * rank <= e < 4 * rank + 4 else -1 for e in range(8)], np.int32)
        sub = dict(m, EL=4, A=[a[:, 4 * rank:4 * rank + 4] for a in m["A"]],
                   B=[b[:, 4 * rank:4 * rank + 4] for b in m["B"]])
        parts = parts + oracle.moe_rows(sub["x"], sub["topk"], sub["ts"], sub["S"], sub["E"], 4, sub["A"],
                                        sub["B"], sub["offsets"], 1.5, sub["y0"], expert_map=emap, add=False,
                                        lib=lib)
    windows = np.zeros(full.shape[1], bool)
    for o, w in zip(m["offsets"], (16, 8)):
        windows[o:o + w] = True
    assert np.array_equal(parts[:, windows], full[:, windows])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
