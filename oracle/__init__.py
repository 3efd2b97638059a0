"""CPU oracle for the multi-LoRA batched low-rank delta (fp64, plain C).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The GPU product path never imports it.

The arithmetic lives in ``lora_oracle.c``; this module only marshals numpy
arrays into that library.  See the header of ``lora_oracle.c`` for what each
function computes and which passage of the pages it follows.

Parity pins: every function here is pinned by tests in ``tests/`` that do not
go through this library's arithmetic (worked examples printed on the pages,
closed forms, invariants, brute force); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

F32, BF16 = 0, 1

_lib = None


def load(path: str | None = None) -> C.CDLL:
    """Load the oracle library, building it first if it is missing."""
    global _lib
    if path is not None:
        lib = C.CDLL(path)
        _declare(lib)
        return lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = C.CDLL(_build.LIB)
        _declare(_lib)
    return _lib


def _declare(lib: C.CDLL) -> None:
    p = C.c_void_p
    i32, i64 = C.c_int32, C.c_int64
    lib.oracle_prepare_meta.argtypes = [p, i64, i32, p, p, p, p, p, p, p]
    lib.oracle_prepare_meta.restype = C.c_int
    lib.oracle_lora_rows.argtypes = [C.c_int, p, i64, i64, p, i32, i32, p, p,
                                     i32, p, p, p, p, C.c_double, p, p, i64,
                                     C.c_int, p, i64, p, p]
    lib.oracle_lora_rows.restype = C.c_int
    lib.oracle_expand_rows.argtypes = [C.c_int, p, i64, p, i32, i32, i32, p, p,
                                       p, p, p, i64, C.c_int, p, i64, p]
    lib.oracle_expand_rows.restype = C.c_int
    lib.oracle_moe_keys.argtypes = [p, i64, i32, p, i32, i32, i32, p, p]
    lib.oracle_moe_keys.restype = C.c_int


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


@dataclass
class Meta:
    sorted: np.ndarray      # int32 [T]
    seg_slot: np.ndarray    # int32 [S+1]
    seg_count: np.ndarray   # int32 [S+1]
    seg_start: np.ndarray   # int32 [S+2]
    num_segments: int
    no_lora: int
    num_bad: int


def prepare_meta(token_slot: np.ndarray, num_slots: int, lib=None) -> Meta:
    lib = lib or load()
    ts = np.ascontiguousarray(token_slot, dtype=np.int32)
    T, S = ts.shape[0], int(num_slots)
    out = dict(sorted=np.zeros(max(T, 1), np.int32),
               seg_slot=np.zeros(S + 1, np.int32),
               seg_count=np.zeros(S + 1, np.int32),
               seg_start=np.zeros(S + 2, np.int32))
    scal = np.zeros(3, np.int32)
    rc = lib.oracle_prepare_meta(_ptr(ts), T, S, _ptr(out["sorted"]),
                                 _ptr(out["seg_slot"]), _ptr(out["seg_count"]),
                                 _ptr(out["seg_start"]), _ptr(scal[0:1]),
                                 _ptr(scal[1:2]), _ptr(scal[2:3]))
    if rc != 0:
        raise ValueError("oracle_prepare_meta rejected its arguments")
    out["sorted"] = out["sorted"][:T]
    return Meta(**out, num_segments=int(scal[0]), no_lora=int(scal[1]),
                num_bad=int(scal[2]))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {a.dtype}")


def lora_rows(x, token_slot, num_slots, A, B, offsets, scale, y0, add=True,
              rows=None, slot_scale=None, return_u=False, lib=None):
    """fp64 rows of ``y0 + s*(x A[slot]) B[slot]`` (see ``oracle_lora_rows``).

    x [T][d_in]; A: list of per-slice arrays [S][d_in][r_max]; B: list of
    per-slice arrays [S][r_max][w_s]; offsets: per-slice column offsets in y0
    [T][ldy].  Floating arrays are float32 or bf16 bit patterns as uint16.
    """
    lib = lib or load()
    x = np.ascontiguousarray(x)
    dt = _dtype_code(x)
    T, d_in = x.shape
    ts = np.ascontiguousarray(token_slot, dtype=np.int32)
    y0 = np.ascontiguousarray(y0)
    ldy = y0.shape[1]
    A = [np.ascontiguousarray(a) for a in A]
    B = [np.ascontiguousarray(b) for b in B]
    for arr in (*A, *B, y0):
        if _dtype_code(arr) != dt:
            raise TypeError("x, A, B and y0 must share one dtype")
    n_slices = len(A)
    r_max = A[0].shape[2]
    a_ptrs = (C.c_void_p * n_slices)(*[a.ctypes.data for a in A])
    b_ptrs = (C.c_void_p * n_slices)(*[b.ctypes.data for b in B])
    a_ss = np.array([a.shape[1] * a.shape[2] for a in A], np.int64)
    b_ss = np.array([b.shape[1] * b.shape[2] for b in B], np.int64)
    width = np.array([b.shape[2] for b in B], np.int64)
    offs = np.array(offsets, np.int64)
    rows = np.arange(T, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    y_out = np.zeros((rows.shape[0], ldy), np.float64)
    u_out = np.zeros((rows.shape[0], n_slices, r_max), np.float64) if return_u else None
    ss = None if slot_scale is None else np.ascontiguousarray(slot_scale, np.float32)
    rc = lib.oracle_lora_rows(dt, _ptr(x), x.shape[1], d_in, _ptr(ts), int(num_slots),
                              n_slices, a_ptrs, _ptr(a_ss), r_max, b_ptrs, _ptr(b_ss),
                              _ptr(width), _ptr(offs), float(scale), _ptr(ss),
                              _ptr(y0), ldy, int(bool(add)), _ptr(rows),
                              rows.shape[0], _ptr(y_out), _ptr(u_out))
    if rc != 0:
        raise ValueError("oracle_lora_rows rejected its arguments")
    return (y_out, u_out) if return_u else y_out


def expand_rows(u, token_slot, num_slots, B, offsets, y0, add=True, rows=None, lib=None):
    """fp64 rows of the expand step from a given fp32 buffer u [n_slices][T][r_max]."""
    lib = lib or load()
    u = np.ascontiguousarray(u, dtype=np.float32)
    n_slices, T, r_max = u.shape
    ts = np.ascontiguousarray(token_slot, dtype=np.int32)
    y0 = np.ascontiguousarray(y0)
    dt = _dtype_code(y0)
    ldy = y0.shape[1]
    B = [np.ascontiguousarray(b) for b in B]
    b_ptrs = (C.c_void_p * n_slices)(*[b.ctypes.data for b in B])
    b_ss = np.array([b.shape[1] * b.shape[2] for b in B], np.int64)
    width = np.array([b.shape[2] for b in B], np.int64)
    offs = np.array(offsets, np.int64)
    rows = np.arange(T, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    y_out = np.zeros((rows.shape[0], ldy), np.float64)
    rc = lib.oracle_expand_rows(dt, _ptr(u), T, _ptr(ts), int(num_slots), n_slices,
                                r_max, b_ptrs, _ptr(b_ss), _ptr(width), _ptr(offs),
                                _ptr(y0), ldy, int(bool(add)), _ptr(rows),
                                rows.shape[0], _ptr(y_out))
    if rc != 0:
        raise ValueError("oracle_expand_rows rejected its arguments")
    return y_out


def moe_keys(topk_ids, token_slot, num_slots, num_experts, num_local_experts, expert_map=None,
             lib=None) -> np.ndarray:
    """Key of every (token, choice) pair (oracle_moe_keys): int32 [T * topk]."""
    lib = lib or load()
    topk_ids = np.ascontiguousarray(topk_ids, np.int32)
    token_slot = np.ascontiguousarray(token_slot, np.int32)
    T, K = topk_ids.shape
    em = None if expert_map is None else np.ascontiguousarray(expert_map, np.int32)
    keys = np.empty(T * K, np.int32)
    rc = lib.oracle_moe_keys(_ptr(topk_ids), T, K, _ptr(token_slot), num_slots, num_experts,
                             num_local_experts, _ptr(em), _ptr(keys))
    assert rc == 0, rc
    return keys


def moe_rows(x, topk_ids, token_slot, num_slots, num_experts, num_local_experts, A, B, offsets,
             scale, y0, expert_map=None, x_per_pair=False, add=True, rows=None, slot_scale=None,
             lib=None):
    """The experts' LoRA of one MoE layer step ([V] section "融合计算:add_lora_w13
    与 add_lora_w2"): output row p = t * topk + j gets the delta of token t's
    adapter on its j-th expert, with the factors of (slot, local expert).  A_s
    and B_s are stacked [S][E_local][...]; the input row of pair p is x[t] (the
    token's hidden state, gate/up LoRA) or x[p] when x_per_pair (down LoRA).
    Evaluated as the rows of lora_rows with the pair keys as slots."""
    lib = lib or load()
    keys = moe_keys(topk_ids, token_slot, num_slots, num_experts, num_local_experts, expert_map, lib)
    K = np.asarray(topk_ids).shape[1]
    xp = x if x_per_pair else np.repeat(x, K, axis=0)
    SE = num_slots * num_local_experts
    Af = [np.ascontiguousarray(a).reshape((SE,) + a.shape[2:]) for a in A]
    Bf = [np.ascontiguousarray(b).reshape((SE,) + b.shape[2:]) for b in B]
    ss = None if slot_scale is None else np.repeat(np.asarray(slot_scale, np.float32), num_local_experts)
    return lora_rows(xp, keys, SE, Af, Bf, offsets, scale, y0, add=add, rows=rows, slot_scale=ss, lib=lib)
