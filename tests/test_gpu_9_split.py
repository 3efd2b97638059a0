"""The split decode kernel: each work tile of a decode-shaped bf16 lora_apply
spread over G workgroups that exchange partial rank rows through memory and
meet at per-tile flag words (page "多 LoRA 服务：分段矩阵乘与适配器调度", section
"不合并权重，批量计算": the fused gather-and-multiply form for decode).  Results
against the oracle's fp64 rows; the flags show that the split path ran, that
every call raised each word of each live tile once, and that no wait gave up."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import TOL, DevCase, check_rows, from_dev, oracle_rows, to_dev

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def L():
    import segmented_gather_rank_amd as lib
    return lib


def decode_case(seed, r, S=32, T=256, d_in=1024, widths=(512, 256, 136), none_frac=0.1, ranks=None):
    """One token per request, slots drawn uniformly, some tokens without an
    adapter; the last slice is 8.5 column blocks wide (a ragged block)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    req = rng.integers(0, S, T).astype(np.int32)
    req[rng.random(T) < none_frac] = -1
    widths = list(widths)
    c = W.make_case(name=f"split_r{r}_s{seed}", seed=seed, rng=rng, dtype="bf16", lengths=np.ones(T, np.int64),
                    req_slot=req, num_slots=S, d_in=d_in, r_max=r, widths=widths, scale=0.5, ranks=ranks,
                    weight_sd=0.05)
    c.slot_scale = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), S)
    return c


def live_tiles(meta):
    """Tile indices with an adapter, and all tile indices, from the metadata."""
    t = {k: v.cpu().numpy() for k, v in meta.tensors().items()}
    n = int(t["info"][4])
    slots = t["tiles"][:n, 0]
    return np.where(slots >= 0)[0], n


def tile_flags(L, d, meta):
    """The count words of the apply workspace d.ws, [tile][range][member],
    as uint32: the call count in bits 31:17 (modulo 2^15), the tile in 16:6,
    the range in 5:4, the XCD that raised the word last in 3:0."""
    n = L.max_tiles(meta.num_tokens, meta.num_slots)
    return L.apply_workspace_flags(d.ws, n).cpu().numpy().view(np.uint32)


def check_counters(L, ws):
    """No wait gave up.  A member that met a peer on another XCD is counted
    and printed, not failed: which XCD runs a workgroup is the dispatcher's
    choice (round robin over blockIdx in every record taken), and such a
    member computes the peer's partials itself, so the results checked before
    this stay exact."""
    cnt = L.apply_workspace_counters(ws)
    if cnt["other_xcd"]:
        print(f"[counters] {cnt}", flush=True)
    assert cnt["gave_up"] == 0, cnt
    return cnt


def check_flags(L, d, meta, calls, ranges=1):
    """Every word of the first `ranges` slice ranges of a live tile counts
    `calls` calls and, unless a member met a peer on another XCD, names one
    XCD (all members of a tile ran on one); the other words were never
    touched; no wait gave up."""
    f = tile_flags(L, d, meta)
    live, n = live_tiles(meta)
    cnt, tag = f >> 17, f & 15
    assert (cnt[live, :ranges] == calls).all(), cnt[live]
    # every raised word names its own tile and range
    assert (((f[live, :ranges] >> 6) & 2047) == live[:, None, None]).all()
    assert (((f[live, :ranges] >> 4) & 3) == np.arange(ranges)[None, :, None]).all()
    assert (f[live, ranges:] == 0).all()
    dead = np.setdiff1d(np.arange(f.shape[0]), live)
    assert (f[dead] == 0).all()
    if check_counters(L, d.ws)["other_xcd"] == 0:
        assert (tag[live, :ranges] == tag[live, :ranges, :1]).all(), tag[live]


@pytest.mark.parametrize("r", [8, 16, 32, 64])
@pytest.mark.parametrize("add", [True, False])
def test_split_decode_parity(L, r, add):
    c = decode_case(500 + r, r, widths=(512, 136) if r == 64 else (512, 256, 136))
    print(f"[split] {c.name} T={c.T} S={c.num_slots} add={add}", flush=True)
    d = DevCase(c)
    y, meta = d.apply(L, mode="auto", add=add)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T), add=add), c.name)
    check_flags(L, d, meta, 1, ranges=len(c.widths))  # the slices run side by side


@pytest.mark.parametrize("d_in,r", [(14336, 16), (3000, 8), (5000, 32), (4096, 64), (1024, 64)])
def test_split_long_rows(L, d_in, r):
    """d_in that splits into 1024-row chunks (rank <= 16) or into chunks that
    do not tile it exactly (the tail of the last member's chunk reads zeros);
    one slice at rank 64."""
    c = decode_case(560 + r, r, d_in=d_in, widths=(1024,))
    print(f"[split-long] {c.name} d_in={d_in}", flush=True)
    d = DevCase(c)
    y, meta = d.apply(L)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), c.name)
    check_flags(L, d, meta, 1)


@pytest.mark.parametrize("r", [16, 32])
def test_split_packed_qkv_decode_shape(L, r):
    """Packed q/k/v of a 4096-wide model at decode (256 tokens, 32 slots):
    three slices side by side, the widest (q, 256 column blocks) setting the
    member count; every slice checked against the oracle."""
    c = decode_case(520 + r, r, d_in=4096, widths=(4096, 1024, 1024))
    print(f"[split-qkv] r={r}", flush=True)
    d = DevCase(c)
    y, meta = d.apply(L)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), c.name)
    check_flags(L, d, meta, 1, ranges=3)


def test_split_rank64_three_slices_side_by_side(L):
    """Three slices at rank 64: each workgroup takes one slice, so the LDS of
    one slice's rank rows is all a workgroup needs."""
    c = decode_case(505, 64)
    d = DevCase(c)
    y, meta = d.apply(L)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), c.name)
    check_flags(L, d, meta, 1, ranges=3)


def test_split_five_slices_rank64_falls_back(L):
    """Five slices at rank 64 fit neither split kernel (at most four slices
    side by side; the packed-slice kernel's LDS): the call runs on the
    one-workgroup-per-token kernel (flags untouched) and is still right."""
    c = decode_case(506, 64, widths=(256, 128, 136, 64, 200))
    d = DevCase(c)
    y, meta = d.apply(L)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), c.name)
    assert (tile_flags(L, d, meta) == 0).all()


def test_split_calls_share_one_meta(L):
    """Calls of different shapes (so different member counts and chunks) on
    one metadata struct, interleaved and repeated: each is right, and the
    flags stay equal across a tile's words."""
    S, T = 32, 256
    shapes = [dict(d_in=1024, widths=(512, 256, 136), r=16), dict(d_in=4096, widths=(4096,), r=16),
              dict(d_in=512, widths=(1024, 1024), r=32), dict(d_in=2048, widths=(8,), r=8)]
    cases = []
    base = decode_case(600, 16, S=S, T=T)
    for i, sh in enumerate(shapes):
        c = decode_case(600, sh["r"], S=S, T=T, d_in=sh["d_in"], widths=sh["widths"])
        assert np.array_equal(c.token_slot, base.token_slot)
        cases.append((c, DevCase(c)))
    meta = L.lora_prepare_meta(cases[0][1].token_slot, S)
    ws = L.apply_workspace(max(L.lora_apply_workspace_bytes(T, S, c.d_in, len(c.widths), c.r_max, torch.bfloat16)
                               for c, _ in cases))
    for rep in range(2):
        for c, d in cases:
            print(f"[split-share] rep {rep} {c.name} d_in={c.d_in} widths={c.widths}", flush=True)
            y, _ = d.apply(L, mode="auto", meta=meta, workspace=ws)
            check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T)), f"{c.name} rep {rep}")
    f = tile_flags(L, cases[0][1], meta)
    live, _ = live_tiles(meta)
    assert ((f[live] >> 4) == (f[live][:, :, :1] >> 4)).all()  # each range's words stay equal
    assert ((f[live, 0] >> 17) >= 2).all()
    check_counters(L, ws)


def test_split_shapes_alternate_on_one_workspace(L):
    """One workspace, calls of four shapes in turn, six rounds: one, two and
    three slices side by side advance their ranges' counts at different
    rates, and the shapes lay the partial fragments out differently, so a
    fragment slot often holds another tile's or range's partials from an
    earlier call with the same count.  The tags name tile and range as well,
    so every call is still right."""
    S, T = 32, 256
    shapes = [dict(d_in=1024, widths=(512, 256, 136), r=16), dict(d_in=2048, widths=(1024, 512), r=16),
              dict(d_in=512, widths=(1024,), r=32), dict(d_in=1024, widths=(256, 256, 256), r=8)]
    base = decode_case(630, 16, S=S, T=T)
    cases = []
    for sh in shapes:
        c = decode_case(630, sh["r"], S=S, T=T, d_in=sh["d_in"], widths=sh["widths"])
        assert np.array_equal(c.token_slot, base.token_slot)
        cases.append((c, DevCase(c), oracle_rows(c, np.arange(c.T))))
    meta = L.lora_prepare_meta(cases[0][1].token_slot, S)
    ws = L.apply_workspace(max(L.lora_apply_workspace_bytes(T, S, c.d_in, len(c.widths), c.r_max, torch.bfloat16)
                               for c, _, _ in cases))
    for rep in range(6):
        for c, d, ref in cases:
            print(f"[split-alt] rep {rep} d_in={c.d_in} widths={c.widths} r={c.r_max}", flush=True)
            y, _ = d.apply(L, mode="auto", meta=meta, workspace=ws)
            check_rows(c, from_dev(y), ref, f"{c.name} rep {rep}")
    check_counters(L, ws)


def test_split_two_streams_one_meta(L):
    """Two decode-shaped applies of different shapes on one lora_meta, at the
    same time on two streams, each call with its own workspace: the metadata is
    only read and the count words live in each call's workspace, so both
    give the oracle's rows, and each stream's repeats are equal bit for bit.
    (With two kernels sharing the CUs, a wait may give up: that case computes
    the same bits, so it is not asserted away.)"""
    S, T = 32, 256
    c1 = decode_case(650, 16, S=S, T=T, d_in=4096, widths=(4096,))
    c2 = decode_case(650, 32, S=S, T=T, d_in=1024, widths=(512, 256, 136))
    assert np.array_equal(c1.token_slot, c2.token_slot)
    d1, d2 = DevCase(c1), DevCase(c2)
    meta = L.lora_prepare_meta(d1.token_slot, S)
    ws = [L.apply_workspace(L.lora_apply_workspace_bytes(T, S, c.d_in, len(c.widths), c.r_max, torch.bfloat16))
          for c in (c1, c2)]
    reps = 6
    ys = [[d.y0.clone() for _ in range(reps)] for d in (d1, d2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    print("[split-2streams] launching", flush=True)
    for i in range(reps):
        for k, d in enumerate((d1, d2)):
            with torch.cuda.stream(streams[k]):
                d.apply(L, meta=meta, y=ys[k][i], workspace=ws[k], stream=streams[k])
    torch.cuda.synchronize()
    for k, c in enumerate((c1, c2)):
        got = [from_dev(y) for y in ys[k]]
        for i in range(1, reps):
            assert np.array_equal(got[i].view(np.uint16), got[0].view(np.uint16)), f"stream {k} rep {i}"
        check_rows(c, got[0], oracle_rows(c, np.arange(c.T)), f"stream {k}")
        print(f"[split-2streams] stream {k}: {L.apply_workspace_counters(ws[k])}", flush=True)
        check_counters(L, ws[k])


def test_split_large_tiles(L):
    """Segments of 17..64 tokens (2..4 token blocks per tile) and longer ones
    cut into several tiles; BGMV mode keeps them on the fused path."""
    rng = np.random.Generator(np.random.PCG64(610))
    lengths = np.array([17, 33, 64, 65, 130, 1, 1, 48, 20], np.int64)
    req = np.array([0, 1, 2, 3, 4, 5, -1, 6, 7], np.int32)
    c = W.make_case(name="split_big_tiles", seed=610, rng=rng, dtype="bf16", lengths=lengths, req_slot=req,
                    num_slots=8, d_in=768, r_max=16, widths=[384, 200], scale=1.0, weight_sd=0.05)
    d = DevCase(c)
    for add in (True, False):
        y, meta = d.apply(L, mode="bgmv", add=add)
        check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T), add=add), f"{c.name} add={add}")
        check_flags(L, d, meta, 1, ranges=2)


@pytest.mark.parametrize("r", [16, 32, 64])
def test_split_large_tiles_one_slice(L, r):
    """The one-slice kernel on tiles of 2..4 token blocks (each wave shrinks
    its own block over the whole chunk) beside one-token tiles (the four
    waves split the chunk), with d_in that the chunks do not tile exactly."""
    rng = np.random.Generator(np.random.PCG64(615 + r))
    lengths = np.array([17, 33, 64, 65, 130, 1, 1, 48, 20, 1, 1, 1], np.int64)
    req = np.array([0, 1, 2, 3, 4, 5, -1, 6, 7, 8, 9, 10], np.int32)
    c = W.make_case(name=f"split_big_tiles_1s_r{r}", seed=615 + r, rng=rng, dtype="bf16", lengths=lengths,
                    req_slot=req, num_slots=12, d_in=1000, r_max=r, widths=[520], scale=1.0, weight_sd=0.05)
    d = DevCase(c)
    for add in (True, False):
        print(f"[split-big-1s] r={r} add={add}", flush=True)
        y, meta = d.apply(L, mode="bgmv", add=add)
        check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T), add=add), f"{c.name} add={add}")
        check_flags(L, d, meta, 1)


@pytest.mark.parametrize("add", [True, False])
def test_split_slot_ranks(L, add):
    """Per-slot ranks, one of them 0: that slot's rows are left as they are
    (add) or cleared (store)."""
    S = 16
    rng = np.random.Generator(np.random.PCG64(620))
    ranks = rng.choice(np.array([0, 8, 16, 24, 32], np.int32), S)
    ranks[3] = 0
    c = decode_case(620, 32, S=S, T=128, ranks=ranks)
    d = DevCase(c)
    y = d.y0.clone()
    meta = L.lora_prepare_meta(d.token_slot, S)
    ws = L.apply_workspace(L.lora_apply_workspace_bytes(c.T, S, c.d_in, len(c.widths), c.r_max, torch.bfloat16))
    L.lora_apply(meta, d.x, d.A, d.B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale, add=add,
                 slot_rank=torch.from_numpy(ranks).cuda(), workspace=ws)
    check_rows(c, from_dev(y), oracle_rows(c, np.arange(c.T), add=add), c.name)
    check_counters(L, ws)


def test_split_graph_replays(L):
    """Metadata and apply captured in one HIP graph: every replay, with eager
    work between them, gives the eager result bit for bit."""
    c = decode_case(630, 16)
    d = DevCase(c)
    y_eager, _ = d.apply(L)
    torch.cuda.synchronize()
    y = d.y0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture (workspace allocations)
        meta = L.lora_prepare_meta(d.token_slot, c.num_slots)
        ws = L.apply_workspace(L.lora_apply_workspace_bytes(c.T, c.num_slots, c.d_in, len(c.widths), c.r_max,
                                                            torch.bfloat16))
    torch.cuda.current_stream().wait_stream(s)
    meta_ws = meta.workspace
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m = L.lora_prepare_meta(d.token_slot, c.num_slots, workspace=meta_ws)
        y.copy_(d.y0)
        L.lora_apply(m, d.x, d.A, d.B, c.offsets, y, scale=c.scale, slot_scale=d.slot_scale, workspace=ws)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i}"
        d.apply(L)  # eager work between replays
        torch.cuda.synchronize()
    check_counters(L, ws)


_FALLBACK_CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[1] + "/tests")
import segmented_gather_rank_amd as L
from test_gpu_9_split import decode_case
from gpu_util import DevCase, from_dev
out = sys.argv[2]
res = {}
for name, args in (("one_slice", dict(seed=640, r=16, widths=(512,))),
                   ("three_slices", dict(seed=641, r=16, widths=(512, 256, 136)))):
    c = decode_case(args["seed"], args["r"], widths=args["widths"])
    d = DevCase(c)
    y, meta = d.apply(L)
    torch.cuda.synchronize()
    res[name] = from_dev(y)
    res[name + "_gave_up"] = np.array([L.apply_workspace_counters(d.ws)["gave_up"]])
np.savez(out, **res)
print("child done", flush=True)
"""


def test_split_fallback_when_peers_are_late(L, tmp_path):
    """With no patience at all (spin limit 0, in a child process: the limit is
    read once per process), members that do not see every peer at their first
    look compute the missing partials themselves.  The results are the normal
    run's, bit for bit."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = str(tmp_path / "fallback.npz")
    env = dict(os.environ, LORA_SPLIT_SPIN_LIMIT="0")
    print("[split-fallback] child process with LORA_SPLIT_SPIN_LIMIT=0", flush=True)
    r = subprocess.run([sys.executable, "-c", _FALLBACK_CHILD, root, out], env=env, capture_output=True,
                       text=True, timeout=100)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    got = np.load(out)
    # the premise: with no patience some member missed a peer and took the
    # fallback (two batches of 33 tiles x 8 members each looked once)
    assert int(got["one_slice_gave_up"][0]) + int(got["three_slices_gave_up"][0]) > 0
    for name, args in (("one_slice", dict(seed=640, r=16, widths=(512,))),
                       ("three_slices", dict(seed=641, r=16, widths=(512, 256, 136)))):
        c = decode_case(args["seed"], args["r"], widths=args["widths"])
        d = DevCase(c)
        y, meta = d.apply(L)
        want = from_dev(y)
        check_counters(L, d.ws)
        print(f"[split-fallback] {name}: {int(got[name + '_gave_up'][0])} waits gave up", flush=True)
        assert np.array_equal(got[name].view(np.uint16), want.view(np.uint16)), name
        check_rows(c, got[name], oracle_rows(c, np.arange(c.T)), f"{name} after fallback")
