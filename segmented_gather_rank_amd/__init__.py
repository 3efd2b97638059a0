"""Python binding of the MI355X multi-LoRA shrink/expand library.

Argument marshalling only: every step of the path runs in the HIP kernels of
``liblora_mi355x.so`` (C ABI in ``include/lora_mi355x.h``).  PyTorch provides
device memory and the current HIP stream.  The functions carry the names of the
C entry points.

There is no fallback: importing this package fails loudly when the built
library is missing (build it with ``python segmented_gather_rank_amd/build.py``
or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LORA_MI355X_LIB names another build of the same library (a measurement
# build, say); by default the in-tree one is loaded
LIB_PATH = os.environ.get("LORA_MI355X_LIB") or os.path.join(_HERE, "liblora_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python segmented_gather_rank_amd/build.py)")

_cdll = C.CDLL(LIB_PATH)

LORA_OK, LORA_ERR_INVALID_ARG, LORA_ERR_UNSUPPORTED, LORA_ERR_WORKSPACE, LORA_ERR_HIP = range(5)
LORA_F32, LORA_BF16 = 0, 1
MODES = {"auto": 0, "bgmv": 1, "sgmv": 2}


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {lora_status_string(status)}")
        self.status = status


class lora_weight(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("slot_stride", C.c_int64), ("layout", C.c_int32), ("reserved", C.c_int32)]


LORA_LAYOUT_DEFAULT, LORA_LAYOUT_RANK_ROWS, LORA_LAYOUT_OUT_ROWS = 0, 1, 2


class lora_meta(C.Structure):
    _fields_ = [("num_tokens", C.c_int64), ("num_slots", C.c_int32), ("x_row_div", C.c_int32),
                ("sorted", C.c_void_p), ("sorted_slot", C.c_void_p), ("seg_slot", C.c_void_p),
                ("seg_count", C.c_void_p),
                ("seg_start", C.c_void_p), ("info", C.c_void_p), ("tiles", C.c_void_p)]


_p, _i32, _i64, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_decl = {
    "lora_abi_version": ([], _i32),
    "lora_status_string": ([_i32], C.c_char_p),
    "lora_meta_workspace_bytes": ([_i64, _i32, C.POINTER(_sz)], _i32),
    "lora_prepare_meta": ([_p, _i64, _i32, _p, _sz, C.POINTER(lora_meta), _p], _i32),
    "lora_moe_meta_workspace_bytes": ([_i64, _i32, _i32, _i32, C.POINTER(_sz)], _i32),
    "lora_prepare_moe_meta": ([_p, _i64, _i32, _p, _i32, _i32, _i32, _p, _p, _sz, C.POINTER(lora_meta), _p],
                              _i32),
    "lora_shrink_workspace_bytes": ([_i64, _i32, _i64, _i32, _i32, _i32, _i32, C.POINTER(_sz)], _i32),
    "lora_shrink": ([C.POINTER(lora_meta), _p, _i64, _i64, _i32, _i32, C.POINTER(lora_weight), _i32,
                     C.c_float, _p, _p, _p, _i32, _p, _sz, _p], _i32),
    "lora_expand": ([C.POINTER(lora_meta), _p, _i32, C.POINTER(lora_weight), C.POINTER(_i64),
                     C.POINTER(_i64), _i32, _p, _p, _i64, _i32, C.c_int, _i32, _p], _i32),
    "lora_apply_workspace_bytes": ([_i64, _i32, _i64, _i32, _i32, _i32, _i32, C.POINTER(_sz)], _i32),
    "lora_apply_workspace_init": ([_p, _sz, _p], _i32),
    "lora_apply_noalloc": ([C.POINTER(lora_meta), _p, _i64, _i64, _i32, _i32, C.POINTER(lora_weight),
                            C.POINTER(lora_weight), C.POINTER(_i64), C.POINTER(_i64), _i32, C.c_float, _p,
                            _p, _p, _i64, C.c_int, _i32, _p], _i32),
    "lora_apply": ([C.POINTER(lora_meta), _p, _i64, _i64, _i32, _i32, C.POINTER(lora_weight),
                    C.POINTER(lora_weight), C.POINTER(_i64), C.POINTER(_i64), _i32, C.c_float, _p,
                    _p, _p, _i64, C.c_int, _i32, _p, _sz, _p], _i32),
}



class _Exact:
    """A C function that takes exactly its declared arguments (ctypes itself
    would silently pass extra ones)."""

    def __init__(self, f):
        self.f, self.n = f, len(f.argtypes)

    def __call__(self, *args):
        if len(args) != self.n:
            raise TypeError(f"{self.f.__name__} takes {self.n} arguments, got {len(args)}")
        return self.f(*args)


class _Lib:
    def __init__(self, cdll, decl):
        for name, (args, res) in decl.items():
            f = getattr(cdll, name)
            f.argtypes, f.restype = args, res
            setattr(self, name, _Exact(f))


_lib = _Lib(_cdll, _decl)

if _lib.lora_abi_version() != 10:
    raise ImportError("liblora_mi355x.so has an unexpected ABI version; rebuild it")


def lora_abi_version() -> int:
    return int(_lib.lora_abi_version())


def lora_status_string(status: int) -> str:
    return _lib.lora_status_string(int(status)).decode()


def _check(fn: str, st: int) -> None:
    if st != LORA_OK:
        raise LoraError(fn, st)


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LORA_F32
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _weights(ws, name: str, inner_shape_ok, layout: int = 0) -> tuple:
    """Per-slice stacked factors [S][rows][cols] -> lora_weight array.  The
    matrices must be contiguous; the slot stride is taken from the tensor."""
    if isinstance(ws, torch.Tensor):
        ws = [ws]
    arr = (lora_weight * len(ws))()
    for i, w in enumerate(ws):
        if w.dim() != 3 or w.stride(2) != 1 or w.stride(1) != w.shape[2]:
            raise ValueError(f"{name}[{i}] must be [S][rows][cols] with contiguous matrices")
        inner_shape_ok(i, w)
        arr[i].ptr = _dev(w, f"{name}[{i}]")
        arr[i].slot_stride = w.stride(0)
        arr[i].layout = layout
    return arr, list(ws)


def _a_weights(A, a_rank_rows: bool):
    """A as [S][d_in][r] (default) or, with a_rank_rows, [S][r][d_in] (the
    rank-major layout); returns the descriptors, the tensors and r."""
    A_arr, A_list = _weights(A, "A", lambda i, w: None, LORA_LAYOUT_RANK_ROWS if a_rank_rows else LORA_LAYOUT_DEFAULT)
    return A_arr, A_list, A_list[0].shape[1] if a_rank_rows else A_list[0].shape[2]


TILE_ROWS = 64          # sorted positions per work tile of the metadata
TILE_INTS = 4 + TILE_ROWS
# the apply workspace's count words (LORA_APPLY_SYNC_BYTES and the two
# counter indices of the C header)
APPLY_SYNC_BYTES = 295168
WAITS_GAVE_UP_WORD = 73728
OTHER_XCD_WORD = 73729
SPLIT_MEMBERS = 16      # count words per work tile and slice range
SPLIT_RANGES = 4        # slice ranges per work tile


def max_tiles(num_tokens: int, num_slots: int) -> int:
    """Capacity of the metadata's work-tile list."""
    return (num_tokens + TILE_ROWS - 1) // TILE_ROWS + num_slots + 1


@dataclass
class LoraMeta:
    """Slot metadata of one batch on the device (see ``lora_meta`` in the C header).

    ``workspace`` owns the device arrays; keep this object alive while kernels
    that use it are in flight."""
    c: lora_meta
    workspace: torch.Tensor

    @property
    def num_tokens(self) -> int:
        return int(self.c.num_tokens)

    @property
    def num_slots(self) -> int:
        return int(self.c.num_slots)

    def _view(self, ptr, n):
        off = ptr - self.workspace.data_ptr()
        return self.workspace[off:off + 4 * n].view(torch.int32)

    def with_x_row_div(self, div: int) -> "LoraMeta":
        """The same metadata with another x row divisor (MoE: 1 for the
        down-projection LoRA, whose input has one row per pair)."""
        c = lora_meta()
        C.pointer(c)[0] = self.c
        c.x_row_div = int(div)
        return LoraMeta(c, self.workspace)

    def tensors(self) -> dict:
        """Device int32 views of the metadata arrays."""
        T, S = self.num_tokens, self.num_slots
        return dict(sorted=self._view(self.c.sorted, T), sorted_slot=self._view(self.c.sorted_slot, T),
                    seg_slot=self._view(self.c.seg_slot, S + 1),
                    seg_count=self._view(self.c.seg_count, S + 1),
                    seg_start=self._view(self.c.seg_start, S + 2), info=self._view(self.c.info, 8),
                    tiles=self._view(self.c.tiles, TILE_INTS * max_tiles(T, S)).view(-1, TILE_INTS))


def lora_meta_workspace_bytes(num_tokens: int, num_slots: int) -> int:
    b = _sz(0)
    _check("lora_meta_workspace_bytes", _lib.lora_meta_workspace_bytes(num_tokens, num_slots, C.byref(b)))
    return int(b.value)


def lora_prepare_meta(token_slot: torch.Tensor, num_slots: int, workspace: torch.Tensor | None = None,
                      stream=None) -> LoraMeta:
    if token_slot.dtype != torch.int32 or token_slot.dim() != 1 or not token_slot.is_contiguous():
        raise ValueError("token_slot must be a contiguous int32 vector")
    T = token_slot.shape[0]
    need = lora_meta_workspace_bytes(T, num_slots)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=token_slot.device)
    m = lora_meta()
    st = _lib.lora_prepare_meta(_dev(token_slot, "token_slot") if T else None, T, num_slots,
                                _dev(workspace, "workspace"), workspace.numel(), C.byref(m), _stream(stream))
    _check("lora_prepare_meta", st)
    return LoraMeta(m, workspace)


def lora_moe_meta_workspace_bytes(num_tokens: int, topk: int, num_slots: int, num_local_experts: int) -> int:
    b = _sz(0)
    _check("lora_moe_meta_workspace_bytes",
           _lib.lora_moe_meta_workspace_bytes(num_tokens, topk, num_slots, num_local_experts, C.byref(b)))
    return int(b.value)


def lora_prepare_moe_meta(topk_ids: torch.Tensor, token_slot: torch.Tensor, num_slots: int, num_experts: int,
                          num_local_experts: int, expert_map: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stream=None) -> LoraMeta:
    """Metadata over the (token, choice) pairs of a top-k routing step, keyed by
    (slot, local expert); topk_ids int32 [T][topk], token_slot int32 [T],
    expert_map int32 [num_experts] or None."""
    for name, t in (("topk_ids", topk_ids), ("token_slot", token_slot)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous int32")
    if topk_ids.dim() != 2 or token_slot.dim() != 1 or topk_ids.shape[0] != token_slot.shape[0]:
        raise ValueError("topk_ids must be [T][topk] and token_slot [T]")
    T, K = topk_ids.shape
    need = lora_moe_meta_workspace_bytes(T, K, num_slots, num_local_experts)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=topk_ids.device)
    em = None
    if expert_map is not None:
        if expert_map.dtype != torch.int32 or expert_map.numel() != num_experts:
            raise ValueError("expert_map must be int32 [num_experts]")
        em = _dev(expert_map, "expert_map")
    m = lora_meta()
    st = _lib.lora_prepare_moe_meta(_dev(topk_ids, "topk_ids") if T else None, T, K,
                                    _dev(token_slot, "token_slot") if T else None, num_slots, num_experts,
                                    num_local_experts, em, _dev(workspace, "workspace"), workspace.numel(),
                                    C.byref(m), _stream(stream))
    _check("lora_prepare_moe_meta", st)
    return LoraMeta(m, workspace)


def lora_shrink_workspace_bytes(num_tokens, num_slots, d_in, n_slices, r_max, dtype, mode="auto") -> int:
    b = _sz(0)
    dt = dtype if isinstance(dtype, int) else _dtype(torch.empty(0, dtype=dtype))
    _check("lora_shrink_workspace_bytes",
           _lib.lora_shrink_workspace_bytes(num_tokens, num_slots, d_in, n_slices, r_max, dt,
                                            MODES[mode], C.byref(b)))
    return int(b.value)


def lora_apply_workspace_bytes(num_tokens, num_slots, d_in, n_slices, r_max, dtype, mode="auto") -> int:
    b = _sz(0)
    dt = dtype if isinstance(dtype, int) else _dtype(torch.empty(0, dtype=dtype))
    _check("lora_apply_workspace_bytes",
           _lib.lora_apply_workspace_bytes(num_tokens, num_slots, d_in, n_slices, r_max, dt,
                                           MODES[mode], C.byref(b)))
    return int(b.value)


def lora_apply_workspace_init(workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Zero the count words at the start of an apply workspace (once,
    before its first lora_apply)."""
    _check("lora_apply_workspace_init",
           _lib.lora_apply_workspace_init(_dev(workspace, "workspace"), workspace.numel(), _stream(stream)))
    return workspace


def apply_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled apply workspace of at least nbytes (and at least the
    count words), ready for lora_apply."""
    return torch.zeros(max(int(nbytes), APPLY_SYNC_BYTES), dtype=torch.uint8, device=device)


def apply_workspace_counters(workspace: torch.Tensor) -> dict:
    """The decode-shaped apply's counters in a workspace: waits that gave up
    and waits that met a peer on another XCD (0 and 0 in normal runs; either
    case is still computed right).  Synchronises with the device."""
    w = workspace[:APPLY_SYNC_BYTES].view(torch.int32)
    v = w[WAITS_GAVE_UP_WORD:OTHER_XCD_WORD + 1].cpu().tolist()
    return {"gave_up": int(v[0]) & 0xFFFFFFFF, "other_xcd": int(v[1]) & 0xFFFFFFFF}


def apply_workspace_flags(workspace: torch.Tensor, tiles: int) -> torch.Tensor:
    """The count words of the first `tiles` work tiles, [tile][range][member]
    (int32 view of uint32 words: the call count in bits 31:17, the tile in
    16:6, the range in 5:4, an XCD in 3:0)."""
    w = workspace[:APPLY_SYNC_BYTES].view(torch.int32)
    return w[:tiles * SPLIT_RANGES * SPLIT_MEMBERS].view(tiles, SPLIT_RANGES, SPLIT_MEMBERS)


def _x_args(x: torch.Tensor):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [T][ldx] with unit column stride")
    return _dev(x, "x"), x.stride(0), x.shape[1]


def _ranks(slot_rank):
    if slot_rank is None:
        return None
    if slot_rank.dtype != torch.int32:
        raise TypeError("slot_rank must be int32")
    return _dev(slot_rank, "slot_rank")


def lora_shrink(meta: LoraMeta, x: torch.Tensor, A, u: torch.Tensor, scale: float = 1.0,
                slot_scale: torch.Tensor | None = None, mode: str = "auto",
                workspace: torch.Tensor | None = None, stream=None,
                slot_rank: torch.Tensor | None = None, a_rank_rows: bool = False) -> torch.Tensor:
    """u[s][t][:] = scale * slot_scale[slot] * x[t] @ A[s][slot]; A: list of [S][d_in][r]
    (or [S][r][d_in] with a_rank_rows).  slot_rank: optional int32 [S], ranks
    each slot's adapter really has."""
    xp, ldx, d_in = _x_args(x)
    A_arr, A_list, r = _a_weights(A, a_rank_rows)
    n = len(A_list)
    need = lora_shrink_workspace_bytes(meta.num_tokens, meta.num_slots, d_in, n, r, x.dtype, mode)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    ss = None if slot_scale is None else _dev(slot_scale, "slot_scale")
    st = _lib.lora_shrink(C.byref(meta.c), xp, ldx, d_in, _dtype(x), n, A_arr, r, float(scale), ss,
                          _ranks(slot_rank), _dev(u, "u"), MODES[mode], _dev(workspace, "workspace"),
                          workspace.numel(), _stream(stream))
    _check("lora_shrink", st)
    return u


def _b_weights(B, b_out_rows: bool):
    """B as [S][r][w] (default) or, with b_out_rows, [S][w][r] (one row of
    ranks per output column); returns the descriptors, the tensors and r."""
    B_arr, B_list = _weights(B, "B", lambda i, w: None, LORA_LAYOUT_OUT_ROWS if b_out_rows else LORA_LAYOUT_DEFAULT)
    return B_arr, B_list, B_list[0].shape[2] if b_out_rows else B_list[0].shape[1]


def _slices(B_list, offsets, b_out_rows: bool = False):
    n = len(B_list)
    width = (C.c_int64 * n)(*[b.shape[1] if b_out_rows else b.shape[2] for b in B_list])
    offs = (C.c_int64 * n)(*[int(o) for o in offsets])
    return width, offs


def lora_expand(meta: LoraMeta, u: torch.Tensor, B, offsets, y: torch.Tensor, add: bool = True,
                mode: str = "auto", stream=None, slot_rank: torch.Tensor | None = None,
                b_out_rows: bool = False) -> torch.Tensor:
    """y[t][off_s:off_s+w_s] (+)= u[s][t] @ B[s][slot]; B: list of [S][r][w_s]
    (or [S][w_s][r] with b_out_rows)."""
    B_arr, B_list, rb = _b_weights(B, b_out_rows)
    width, offs = _slices(B_list, offsets, b_out_rows)
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be [T][ldy] with unit column stride")
    st = _lib.lora_expand(C.byref(meta.c), _dev(u, "u"), len(B_list), B_arr, width, offs,
                          rb, _ranks(slot_rank), _dev(y, "y"), y.stride(0), _dtype(y),
                          int(bool(add)), MODES[mode], _stream(stream))
    _check("lora_expand", st)
    return y


def lora_apply(meta: LoraMeta, x: torch.Tensor, A, B, offsets, y: torch.Tensor, scale: float = 1.0,
               slot_scale: torch.Tensor | None = None, add: bool = True, mode: str = "auto",
               workspace: torch.Tensor | None = None, stream=None,
               slot_rank: torch.Tensor | None = None, a_rank_rows: bool = False,
               b_out_rows: bool = False) -> torch.Tensor:
    """Shrink then expand into the slices of y (the whole delta of one layer).
    A: list of [S][d_in][r], or [S][r][d_in] with a_rank_rows; B: list of
    [S][r][w_s], or [S][w_s][r] with b_out_rows."""
    xp, ldx, d_in = _x_args(x)
    A_arr, A_list, r = _a_weights(A, a_rank_rows)
    B_arr, B_list, _ = _b_weights(B, b_out_rows)
    width, offs = _slices(B_list, offsets, b_out_rows)
    n = len(A_list)
    if len(B_list) != n:
        raise ValueError("A and B need one entry per slice")
    need = lora_apply_workspace_bytes(meta.num_tokens, meta.num_slots, d_in, n, r, x.dtype, mode)
    if workspace is None:
        workspace = apply_workspace(need, x.device)
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be [T][ldy] with unit column stride")
    ss = None if slot_scale is None else _dev(slot_scale, "slot_scale")
    if y.dtype != x.dtype:
        raise TypeError("x and y must share one dtype")
    st = _lib.lora_apply(C.byref(meta.c), xp, ldx, d_in, _dtype(x), n, A_arr, B_arr, width, offs, r,
                         float(scale), ss, _ranks(slot_rank), _dev(y, "y"), y.stride(0), int(bool(add)),
                         MODES[mode], _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check("lora_apply", st)
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20   # LORA_NOALLOC_SCRATCH_BYTES of the C header


def lora_apply_noalloc(meta: LoraMeta, x: torch.Tensor, A, B, offsets, y: torch.Tensor, scale: float = 1.0,
                       slot_scale: torch.Tensor | None = None, add: bool = True, mode: str = "auto", stream=None,
                       slot_rank: torch.Tensor | None = None, a_rank_rows: bool = False,
                       b_out_rows: bool = False) -> torch.Tensor:
    """lora_apply with the library's own device scratch as its workspace (no
    workspace argument, nothing allocated).  Calls that overlap on one device
    share that scratch and race."""
    xp, ldx, d_in = _x_args(x)
    A_arr, A_list, r = _a_weights(A, a_rank_rows)
    B_arr, B_list, _ = _b_weights(B, b_out_rows)
    width, offs = _slices(B_list, offsets, b_out_rows)
    if len(B_list) != len(A_list):
        raise ValueError("A and B need one entry per slice")
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be [T][ldy] with unit column stride")
    if y.dtype != x.dtype:
        raise TypeError("x and y must share one dtype")
    ss = None if slot_scale is None else _dev(slot_scale, "slot_scale")
    st = _lib.lora_apply_noalloc(C.byref(meta.c), xp, ldx, d_in, _dtype(x), len(A_list), A_arr, B_arr, width,
                                 offs, r, float(scale), ss, _ranks(slot_rank), _dev(y, "y"),
                                 y.stride(0), int(bool(add)), MODES[mode], _stream(stream))
    _check("lora_apply_noalloc", st)
    return y


__all__ = ["lora_apply_noalloc", "NOALLOC_SCRATCH_BYTES", "lora_abi_version", "lora_status_string", "lora_meta_workspace_bytes", "lora_prepare_meta",
           "lora_moe_meta_workspace_bytes", "lora_prepare_moe_meta",
           "lora_shrink_workspace_bytes", "lora_shrink", "lora_expand", "lora_apply_workspace_bytes",
           "lora_apply_workspace_init", "apply_workspace", "apply_workspace_counters", "apply_workspace_flags",
           "lora_apply", "LoraMeta", "LoraError", "lora_weight", "lora_meta", "LIB_PATH", "LORA_LAYOUT_DEFAULT",
           "LORA_LAYOUT_RANK_ROWS", "LORA_LAYOUT_OUT_ROWS"]
