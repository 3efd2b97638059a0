"""Seeded synthetic inputs for the multi-LoRA shrink/expand path.

This module only draws and lays out inputs: request structure, slot ids,
activations, adapter factors and the base output.  It holds none of the
method's arithmetic, and both the GPU path (through the tests and the
benchmark) and the CPU oracle read the arrays it returns.

Floating inputs are drawn in float32 and, for bf16 workloads, rounded once
(round to nearest even) to bf16 here, so that both sides see the same bits.
bf16 arrays are returned as their uint16 bit patterns.

Workloads (shapes and distributions of the five standard cases):
  1 toy fp32        -- the handbook's runnable toy ("多 LoRA 服务：分段矩阵乘与适配器调度",
                       section "不合并权重，批量计算"): 8 slots, d=256, r=16,
                       6 requests of lengths [1,1,37,1,12,1] on slots
                       [3,5,3,0,7,5], scale 2.0; drawn with torch.manual_seed(0)
                       in the order W, A, B, x as on that page.
  2 decode bf16     -- q_proj 4096 -> 4096, r=16, 32 slots, 256 one-token
                       requests, 10% without adapter, scale 32/16.
  3 prefill bf16    -- gate_up 4096 -> 2 x 14336, r=64, 8 slots, 16 requests of
                       length U{128..2048}, scale 64/64.
  4 mixed qkv bf16  -- 4096 -> q 4096 / k 1024 / v 1024, r_max=32 with slot
                       ranks U{8,16,32} zero-padded, 64 slots, 512 one-token
                       requests then 4 requests of 1024, slots Zipf(1.1),
                       scale alpha/r = 2.
  5 many-adapter    -- down_proj 14336 -> 4096, r_max=64 with slot ranks
                       U{8,16,32,64}, 128 slots, 4096 one-token requests,
                       slots Zipf(0.8), 5% without adapter, scale 1.0.
  6 logits          -- the LoRA of the vocabulary projection on the rows the
                       sampler reads ("vLLM 源码完全拆解(十八):多 LoRA 服务",
                       section "lm_head / logits"): a step of 192 decode
                       requests and 8 prefill requests of length U{64..1024}
                       samples one row per request (the last one); those 200
                       rows, with the slots of their requests, are the batch.
                       4096 -> vocabulary 76 800 (the vocabulary size of that
                       page's embedding example), r=16, 8 slots, 10 requests
                       without adapter, scale 2.
  7 MoE gate/up     -- the experts' LoRA of a top-8 MoE layer in a decode step
                       ("vLLM 源码完全拆解(十八)", section "MoE 的 LoRA:按专家
                       挂载、融合 kernel 与 EP 切片", its buffer list: hidden
                       7168, expert intermediate 2048, 256 experts, 8-way
                       expert parallelism so 32 local experts, rank 64, 4
                       slots): 256 tokens, 8 distinct experts each, uniform;
                       the rank-0 shard holds experts 0..31.  Gate and up
                       slices (2048 each) of the 2048 (token, choice) rows;
                       x is the tokens' hidden state.  Scale 1 (the page gives
                       no alpha).
  8 MoE down        -- the same step's down-projection LoRA: x has one row
                       per (token, choice) pair (the activated intermediate,
                       2048 wide), output 7168.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------- bf16


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def to_f32(a: np.ndarray) -> np.ndarray:
    """float32 view of a workload array of either dtype."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


# --------------------------------------------------------------------------- case


@dataclass
class Case:
    name: str
    dtype: str                      # "f32" or "bf16"
    lengths: np.ndarray             # int64 [n_requests]
    req_slot: np.ndarray            # int32 [n_requests]
    token_slot: np.ndarray          # int32 [T]
    num_slots: int
    d_in: int
    r_max: int
    ranks: np.ndarray               # int32 [S], rank of each slot's adapter
    widths: list                    # per slice
    offsets: list                   # per slice
    ldy: int
    scale: float
    x: np.ndarray                   # [T][d_in]
    A: list                         # per slice [S][d_in][r_max]
    B: list                         # per slice [S][r_max][w_s]
    y0: np.ndarray                  # [T][ldy]
    slot_scale: np.ndarray | None = None
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.token_slot.shape[0])

    @property
    def n_slices(self) -> int:
        return len(self.widths)


# --------------------------------------------------------------------------- draws


def _normal(rng: np.random.Generator, shape, sd: float) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if sd != 1.0:
        out *= np.float32(sd)
    return out


def _draw(rng, shape, sd, dtype):
    """N(0, sd^2) draws in float32, rounded to bf16 bits for bf16 workloads.

    Large arrays are drawn in row blocks to bound host memory."""
    shape = tuple(int(s) for s in shape)
    if dtype == "f32":
        return _normal(rng, shape, sd)
    out = np.empty(shape, np.uint16)
    flat = out.reshape(shape[0], -1)
    rows_per = max(1, (1 << 24) // max(1, flat.shape[1]))
    for r0 in range(0, flat.shape[0], rows_per):
        r1 = min(flat.shape[0], r0 + rows_per)
        flat[r0:r1] = bf16_round(_normal(rng, (r1 - r0, flat.shape[1]), sd))
    return out


def zipf_slots(rng: np.random.Generator, n: int, num_slots: int, s: float) -> np.ndarray:
    """n draws from the finite Zipf law P(i) ~ (i+1)^-s over i = 0..num_slots-1,
    by inverse CDF of uniform draws."""
    p = np.arange(1, num_slots + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p / p.sum())
    cdf[-1] = 1.0
    return np.minimum(np.searchsorted(cdf, rng.random(n), side="right"),
                      num_slots - 1).astype(np.int32)


def expand_requests(lengths, req_slot) -> np.ndarray:
    """Per-token slot ids from per-request lengths and slots (request order kept)."""
    return np.repeat(np.asarray(req_slot, np.int32), np.asarray(lengths, np.int64))


def mark_no_lora(rng, token_slot: np.ndarray, frac: float) -> np.ndarray:
    """Set exactly round(frac*T) tokens, chosen by a seeded permutation, to -1."""
    ts = token_slot.copy()
    k = int(round(frac * ts.shape[0]))
    if k:
        ts[rng.permutation(ts.shape[0])[:k]] = -1
    return ts


def make_case(*, name, seed, dtype, lengths, req_slot, num_slots, d_in, r_max,
              widths, offsets=None, ldy=None, scale=1.0, ranks=None,
              no_lora_frac=0.0, weight_sd=0.02, x_sd=1.0, y_sd=1.0,
              token_slot=None, rng=None) -> Case:
    """Draw one case.  Draw order after the structure: x, A (all slices), B
    (slice by slice), y0.  Slot ranks below r_max are zero-padded: columns
    j >= rank of A and rows j >= rank of B are 0 for that slot."""
    rng = rng or np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, np.int64)
    req_slot = np.asarray(req_slot, np.int32)
    if token_slot is None:
        token_slot = expand_requests(lengths, req_slot)
        if no_lora_frac:
            token_slot = mark_no_lora(rng, token_slot, no_lora_frac)
    token_slot = np.ascontiguousarray(token_slot, np.int32)
    T = token_slot.shape[0]
    widths = [int(w) for w in widths]
    if offsets is None:
        offsets = list(np.concatenate([[0], np.cumsum(widths)[:-1]]).astype(int))
    offsets = [int(o) for o in offsets]
    ldy = int(ldy if ldy is not None else offsets[-1] + widths[-1])
    ranks = (np.full(num_slots, r_max, np.int32) if ranks is None
             else np.asarray(ranks, np.int32))

    x = _draw(rng, (T, d_in), x_sd, dtype)
    A_all = _draw(rng, (num_slots, len(widths), d_in, r_max), weight_sd, dtype)
    B = [_draw(rng, (num_slots, r_max, w), weight_sd, dtype) for w in widths]
    y0 = _draw(rng, (T, ldy), y_sd, dtype)
    A = [np.ascontiguousarray(A_all[:, s]) for s in range(len(widths))]
    for a in range(num_slots):
        ra = int(ranks[a])
        if ra < r_max:
            for s in range(len(widths)):
                A[s][a, :, ra:] = 0
                B[s][a, ra:, :] = 0
    return Case(name=name, dtype=dtype, lengths=lengths, req_slot=req_slot,
                token_slot=token_slot, num_slots=num_slots, d_in=d_in,
                r_max=r_max, ranks=ranks, widths=widths, offsets=offsets,
                ldy=ldy, scale=float(scale), x=x, A=A, B=B, y0=y0, seed=seed)


# --------------------------------------------------------------------------- the five workloads

CONFIG_NAMES = {
    1: "toy_mixed_fp32",
    2: "decode_bgmv_bf16_q4096_r16_s32_t256",
    3: "prefill_sgmv_bf16_gateup4096x2x14336_r64_s8",
    4: "mixed_qkv_gqa_bf16_r32_s64_t4608",
    5: "many_adapter_decode_bf16_down14336x4096_r64_s128_t4096",
    6: "logits_sampled_rows_bf16_d4096_v76800_r16_s8_t200",
    7: "moe_w13_bf16_h7168_i2048_e256ep8_top8_r64_s4_t256",
    8: "moe_w2_bf16_i2048_h7168_e256ep8_top8_r64_s4_t256",
}


@dataclass
class MoeCase:
    """One MoE layer step: token slots, top-k expert choices, the expert map of
    this rank, and factors stacked per (slot, local expert).  Output rows are
    the (token, choice) pairs, row t * topk + j."""
    name: str
    dtype: str
    token_slot: np.ndarray          # int32 [T] (per token)
    topk_ids: np.ndarray            # int32 [T][topk]
    expert_map: np.ndarray | None   # int32 [E_global] or None
    num_slots: int
    num_experts: int
    num_local_experts: int
    d_in: int
    r_max: int
    ranks: np.ndarray               # int32 [S]
    widths: list
    offsets: list
    ldy: int
    scale: float
    x: np.ndarray                   # [T][d_in] (x_per_pair False) or [T*topk][d_in]
    x_per_pair: bool
    A: list                         # per slice [S][E_local][d_in][r_max]
    B: list                         # per slice [S][E_local][r_max][w_s]
    y0: np.ndarray                  # [T*topk][ldy]
    slot_scale: np.ndarray | None = None
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def T(self) -> int:             # tokens
        return int(self.token_slot.shape[0])

    @property
    def topk(self) -> int:
        return int(self.topk_ids.shape[1])

    @property
    def rows(self) -> int:          # (token, choice) pairs
        return self.T * self.topk

    @property
    def n_slices(self) -> int:
        return len(self.A)


def _moe_case(k: int) -> MoeCase:
    seed = 1000 + k
    rng = np.random.Generator(np.random.PCG64(seed))
    T, K, S, E, EL, r = 256, 8, 4, 256, 32, 64
    hidden, inter = 7168, 2048
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ts = rng.integers(0, S, T).astype(np.int32)
    ts[rng.permutation(T)[:26]] = -1
    emap = np.where(np.arange(E) < EL, np.arange(E), -1).astype(np.int32)
    if k == 7:
        d_in, widths, offsets, ldy, per_pair = hidden, [inter, inter], [0, inter], 2 * inter, False
    else:
        d_in, widths, offsets, ldy, per_pair = inter, [hidden], [0], hidden, True
    xr = T * K if per_pair else T
    x = _draw(rng, (xr, d_in), 1.0, "bf16")
    A = [_draw(rng, (S, EL, d_in, r), 0.02, "bf16") for _ in widths]
    B = [_draw(rng, (S, EL, r, w), 0.02, "bf16") for w in widths]
    y0 = _draw(rng, (T * K, ldy), 1.0, "bf16")
    return MoeCase(name=CONFIG_NAMES[k], dtype="bf16", token_slot=ts, topk_ids=topk, expert_map=emap,
                   num_slots=S, num_experts=E, num_local_experts=EL, d_in=d_in, r_max=r,
                   ranks=np.full(S, r, np.int32), widths=widths, offsets=offsets, ldy=ldy, scale=1.0,
                   x=x, x_per_pair=per_pair, A=A, B=B, y0=y0, seed=seed)


def sampler_rows(lengths) -> np.ndarray:
    """Index, in the step's token batch, of the row the sampler reads for each
    request: its last row (one row for a decode request)."""
    return np.cumsum(np.asarray(lengths, np.int64)) - 1


def _toy() -> Case:
    """The handbook toy, drawn exactly as the page draws it (torch CPU RNG,
    seed 0, order W, A, B, x).  y0 is the base product x*W, evaluated in fp64
    and rounded once to fp32: the base layer's output that the LoRA delta is
    added into."""
    import torch

    g = torch.Generator().manual_seed(0)
    d, r, S = 256, 16, 8
    W = torch.randn(d, d, generator=g) / 16
    A = torch.randn(S, d, r, generator=g) / 16
    B = torch.randn(S, r, d, generator=g) / 4
    lengths, slots = [1, 1, 37, 1, 12, 1], [3, 5, 3, 0, 7, 5]
    x = torch.randn(sum(lengths), d, generator=g)
    x_np, W_np = x.numpy().astype(np.float32), W.numpy().astype(np.float32)
    y0 = (x_np.astype(np.float64) @ W_np.astype(np.float64)).astype(np.float32)
    c = Case(name=CONFIG_NAMES[1], dtype="f32", lengths=np.array(lengths, np.int64),
             req_slot=np.array(slots, np.int32),
             token_slot=expand_requests(lengths, slots), num_slots=S, d_in=d,
             r_max=r, ranks=np.full(S, r, np.int32), widths=[d], offsets=[0],
             ldy=d, scale=2.0, x=x_np, A=[A.numpy().astype(np.float32)],
             B=[B.numpy().astype(np.float32)], y0=y0, seed=0)
    c.notes["W"] = W_np
    return c


def config(k: int) -> Case:
    """Workload k (1..5) at its full size."""
    if k == 1:
        return _toy()
    seed = 1000 + k
    rng = np.random.Generator(np.random.PCG64(seed))
    if k == 2:
        S = 32
        return make_case(name=CONFIG_NAMES[2], seed=seed, rng=rng, dtype="bf16",
                         lengths=np.ones(256, np.int64),
                         req_slot=rng.integers(0, S, 256).astype(np.int32),
                         num_slots=S, d_in=4096, r_max=16, widths=[4096],
                         scale=32 / 16, no_lora_frac=0.10)
    if k == 3:
        S = 8
        lengths = rng.integers(128, 2049, 16)
        return make_case(name=CONFIG_NAMES[3], seed=seed, rng=rng, dtype="bf16",
                         lengths=lengths,
                         req_slot=rng.integers(0, S, 16).astype(np.int32),
                         num_slots=S, d_in=4096, r_max=64, widths=[14336, 14336],
                         scale=64 / 64)
    if k == 4:
        S = 64
        lengths = np.concatenate([np.ones(512, np.int64), np.full(4, 1024, np.int64)])
        req_slot = zipf_slots(rng, lengths.shape[0], S, 1.1)
        ranks = rng.choice(np.array([8, 16, 32], np.int32), S)
        return make_case(name=CONFIG_NAMES[4], seed=seed, rng=rng, dtype="bf16",
                         lengths=lengths, req_slot=req_slot, num_slots=S,
                         d_in=4096, r_max=32, widths=[4096, 1024, 1024],
                         offsets=[0, 4096, 5120], ldy=6144, scale=2.0, ranks=ranks)
    if k == 5:
        S = 128
        req_slot = zipf_slots(rng, 4096, S, 0.8)
        ranks = rng.choice(np.array([8, 16, 32, 64], np.int32), S)
        return make_case(name=CONFIG_NAMES[5], seed=seed, rng=rng, dtype="bf16",
                         lengths=np.ones(4096, np.int64), req_slot=req_slot,
                         num_slots=S, d_in=14336, r_max=64, widths=[4096],
                         scale=1.0, ranks=ranks, no_lora_frac=0.05)
    if k == 6:
        S = 8
        step_lengths = np.concatenate([np.ones(192, np.int64), rng.integers(64, 1025, 8)])
        req_slot = rng.integers(0, S, step_lengths.shape[0]).astype(np.int32)
        req_slot[rng.permutation(step_lengths.shape[0])[:10]] = -1
        c = make_case(name=CONFIG_NAMES[6], seed=seed, rng=rng, dtype="bf16",
                      lengths=np.ones(step_lengths.shape[0], np.int64), req_slot=req_slot,
                      num_slots=S, d_in=4096, r_max=16, widths=[76800], scale=2.0)
        c.notes["step_lengths"] = step_lengths
        c.notes["sampled_token_rows"] = sampler_rows(step_lengths)
        return c
    if k in (7, 8):
        return _moe_case(k)
    raise ValueError(f"no workload {k}")
