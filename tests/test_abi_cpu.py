"""The C-ABI library without a GPU: it loads, exports every function the
public header declares, and rejects bad arguments with the documented status
before any HIP call (so these calls never touch a device)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")

import segmented_gather_rank_amd as L  # noqa: E402  (fails loudly if the library is not built)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \t\*]*?\b(lora_\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 9, names
    lib = C.CDLL(L.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert L.lora_abi_version() == 10
    assert L.lora_status_string(0) == "LORA_OK"
    assert L.lora_status_string(3) == "LORA_ERR_WORKSPACE"
    assert L.lora_status_string(99) == "LORA_ERR_UNKNOWN"


def test_workspace_sizes():
    assert L.lora_meta_workspace_bytes(256, 32) >= 4 * (2 * 256 + 33 + 33 + 34 + 8 + 68 * (4 + 33))
    assert L.lora_meta_workspace_bytes(0, 1) > 0
    import torch
    b_apply = L.lora_apply_workspace_bytes(4096, 128, 14336, 1, 64, torch.bfloat16)
    assert b_apply >= L.APPLY_SYNC_BYTES + 4 * 4096 * 64
    # every apply workspace starts with the count words, whatever the call
    assert L.lora_apply_workspace_bytes(1, 1, 8, 1, 8, torch.float32) >= L.APPLY_SYNC_BYTES
    b2 = L.lora_shrink_workspace_bytes(256, 32, 4096, 1, 16, torch.bfloat16)
    assert b2 > 0 and b2 % 256 == 0


def test_workspace_sizes_follow_the_tile_rank():
    """r_max that is not a power of two runs at the next of 8, 16, 32, 64, 128:
    the shrink's partial sums and lora_apply's rank buffer are sized at that
    rank, so r_max = 24 needs the shrink workspace of r_max = 32 and 48 that of
    64.  lora_apply's may be smaller than at the power of two (the fused decode
    kernels, which take only 8, 16, 32 and 64, add their partials there)."""
    import torch
    for T, S, d_in, n in ((4096, 32, 4096, 1), (17705, 4, 4096, 2), (64, 64, 14336, 3)):
        for dt in (torch.bfloat16, torch.float32):
            for lo, hi in ((24, 32), (40, 64), (48, 64), (72, 128), (120, 128)):
                assert L.lora_shrink_workspace_bytes(T, S, d_in, n, lo, dt) == \
                    L.lora_shrink_workspace_bytes(T, S, d_in, n, hi, dt), (T, lo, dt)
                a = L.lora_apply_workspace_bytes(T, S, d_in, n, lo, dt)
                assert L.APPLY_SYNC_BYTES + 4 * n * T * hi <= a <= \
                    L.lora_apply_workspace_bytes(T, S, d_in, n, hi, dt), (T, lo, dt)
    assert L.lora_apply_workspace_bytes(4096, 32, 4096, 1, 128, torch.bfloat16) >= \
        L.APPLY_SYNC_BYTES + 4 * 4096 * 128


def test_header_constants_match_binding():
    """The binding's copies of the header's #define values, and the layout
    they imply: a row of 64 words per possible work tile (1152 of them), then
    the counters."""
    text = open(HEADER).read()
    d = {k: int(v) for k, v in re.findall(r"#define\s+(LORA_\w+)\s+(\d+)", text)}
    assert d["LORA_APPLY_SYNC_BYTES"] == L.APPLY_SYNC_BYTES
    assert d["LORA_APPLY_WAITS_GAVE_UP_WORD"] == L.WAITS_GAVE_UP_WORD
    assert d["LORA_APPLY_OTHER_XCD_WORD"] == L.OTHER_XCD_WORD
    tiles = (8192 + 63) // 64 + 1023 + 1
    assert L.WAITS_GAVE_UP_WORD == tiles * L.SPLIT_RANGES * L.SPLIT_MEMBERS
    assert L.APPLY_SYNC_BYTES == 4 * (tiles + 1) * L.SPLIT_RANGES * L.SPLIT_MEMBERS


_buf = (C.c_uint8 * (1 << 20))()
_base = (C.addressof(_buf) + 255) // 256 * 256


def _ptr(off=0):
    return C.c_void_p(_base + off)


def _call(name, *args):
    return getattr(L._lib, name)(*args)


def test_meta_rejections():
    m = L.lora_meta()
    sz = C.c_size_t(0)
    assert _call("lora_meta_workspace_bytes", -1, 4, C.byref(sz)) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_meta_workspace_bytes", 10, 0, C.byref(sz)) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_meta_workspace_bytes", 10, 1024, C.byref(sz)) == L.LORA_ERR_UNSUPPORTED
    assert _call("lora_prepare_meta", _ptr(), 10, 4, _ptr(), 16, C.byref(m), None) == L.LORA_ERR_WORKSPACE
    assert _call("lora_prepare_meta", None, 10, 4, _ptr(), 1 << 15, C.byref(m), None) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_prepare_meta", _ptr(), 10, 4, _ptr(4), 1 << 15, C.byref(m), None) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_prepare_meta", _ptr(), 10, 4, _ptr(), 1 << 15, None, None) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_prepare_meta", _ptr(), 10, 2000, _ptr(), 1 << 15, C.byref(m), None) == L.LORA_ERR_UNSUPPORTED


def _meta(T=16, S=4):
    m = L.lora_meta()
    m.num_tokens, m.num_slots, m.x_row_div = T, S, 1
    for f in ("sorted", "sorted_slot", "seg_slot", "seg_count", "seg_start", "info", "tiles"):
        setattr(m, f, _base)
    return m


def _w(n, stride):
    arr = (L.lora_weight * n)()
    for i in range(n):
        arr[i].ptr, arr[i].slot_stride = _base, stride
    return arr


def _shrink(meta=None, ldx=64, d_in=64, dtype=1, n=1, A=None, r=16, ss=None, u=None, mode=0,
            ws=None, ws_bytes=1 << 15):
    meta = meta if meta is not None else _meta()
    A = A if A is not None else _w(n, d_in * r)
    return _call("lora_shrink", C.byref(meta), _ptr(), ldx, d_in, dtype, n, A, r, C.c_float(1.0),
                 ss, None, u if u is not None else _ptr(), mode, ws if ws is not None else _ptr(), ws_bytes,
                 None)


def test_shrink_rejections():
    assert _shrink(r=12) == L.LORA_ERR_UNSUPPORTED      # not a multiple of 8
    assert _shrink(r=136) == L.LORA_ERR_UNSUPPORTED     # past 128
    assert _shrink(r=0) == L.LORA_ERR_UNSUPPORTED
    assert _shrink(r=24, A=_w(1, 64 * 24 - 8)) == L.LORA_ERR_INVALID_ARG   # A slots sized for r_max = 24
    assert _shrink(n=0, A=_w(1, 64 * 16)) == L.LORA_ERR_UNSUPPORTED
    assert _shrink(n=9, A=_w(9, 64 * 16)) == L.LORA_ERR_UNSUPPORTED
    assert _shrink(dtype=7) == L.LORA_ERR_UNSUPPORTED
    assert _shrink(mode=5) == L.LORA_ERR_UNSUPPORTED
    assert _shrink(d_in=60, ldx=64, A=_w(1, 64 * 16)) == L.LORA_ERR_INVALID_ARG
    assert _shrink(ldx=60) == L.LORA_ERR_INVALID_ARG
    assert _shrink(A=_w(1, 64 * 16 - 8)) == L.LORA_ERR_INVALID_ARG        # slots overlap
    assert _shrink(u=_ptr(8)) == L.LORA_ERR_INVALID_ARG                    # misaligned
    bad = _meta()
    bad.seg_start = None
    assert _shrink(meta=bad) == L.LORA_ERR_INVALID_ARG
    bad = _meta()
    bad.tiles = None
    assert _shrink(meta=bad) == L.LORA_ERR_INVALID_ARG
    assert _shrink(meta=_meta(T=-1)) == L.LORA_ERR_INVALID_ARG
    # workspace too small: ask for one that needs partial sums
    need = L.lora_shrink_workspace_bytes(4096, 32, 4096, 1, 16, 1)
    assert need > 0
    assert _shrink(meta=_meta(T=4096, S=32), d_in=4096, ldx=4096, A=_w(1, 4096 * 16),
                   ws_bytes=need - 1) == L.LORA_ERR_WORKSPACE


def _expand(n=2, widths=(64, 32), offsets=(0, 64), r=16, ldy=96, B=None, y=None, mode=0, dtype=1):
    wd = (C.c_int64 * n)(*widths[:n])
    of = (C.c_int64 * n)(*offsets[:n])
    B = B if B is not None else (L.lora_weight * n)(*[L.lora_weight(_base, r * w) for w in widths[:n]])
    return _call("lora_expand", C.byref(_meta()), _ptr(), n, B, wd, of, r, None,
                 y if y is not None else _ptr(), ldy, dtype, 1, mode, None)


def test_layout_rejections():
    """Rank-major A ([r][d_in]) is read by the matrix-core shrink only: bf16,
    r_max >= 16, mode AUTO or SGMV, every slice alike.  Output-rows B
    ([w][r]) by the matrix-core expand only: bf16, r_max <= 64, mode AUTO or
    SGMV, every slice alike.  Neither layout is taken by the other factor."""
    def A_rows(n=1, layouts=(1,), stride=64 * 16):
        arr = (L.lora_weight * n)()
        for i in range(n):
            arr[i].ptr, arr[i].slot_stride, arr[i].layout = _base, stride, layouts[min(i, len(layouts) - 1)]
        return arr
    assert _shrink(A=A_rows(), dtype=0) == L.LORA_ERR_UNSUPPORTED          # fp32
    assert _shrink(A=A_rows(), mode=1) == L.LORA_ERR_UNSUPPORTED           # BGMV
    assert _shrink(A=A_rows(stride=64 * 8), r=8) == L.LORA_ERR_UNSUPPORTED  # r_max 8
    assert _shrink(A=A_rows(2, (1, 0)), n=2) == L.LORA_ERR_INVALID_ARG     # slices differ
    assert _shrink(A=A_rows(layouts=(7,))) == L.LORA_ERR_UNSUPPORTED
    assert _shrink(A=A_rows(layouts=(L.LORA_LAYOUT_OUT_ROWS,))) == L.LORA_ERR_UNSUPPORTED
    def B_rows(layouts, r=16, widths=(64, 32)):
        return (L.lora_weight * 2)(*[L.lora_weight(_base, r * w, layouts[min(i, len(layouts) - 1)])
                                     for i, w in enumerate(widths)])
    out = L.LORA_LAYOUT_OUT_ROWS
    assert _expand(B=B_rows((0, out))) == L.LORA_ERR_INVALID_ARG             # slices differ
    assert _expand(B=B_rows((L.LORA_LAYOUT_RANK_ROWS,))) == L.LORA_ERR_UNSUPPORTED
    assert _expand(B=B_rows((7,))) == L.LORA_ERR_UNSUPPORTED
    assert _expand(B=B_rows((out,)), dtype=0) == L.LORA_ERR_UNSUPPORTED     # fp32
    assert _expand(B=B_rows((out,)), mode=1) == L.LORA_ERR_UNSUPPORTED      # BGMV
    assert _expand(B=B_rows((out,), r=128), r=128) == L.LORA_ERR_UNSUPPORTED  # past the tile expand's 64
    thin = (L.lora_weight * 2)(L.lora_weight(_base, 16 * 64 - 8, out), L.lora_weight(_base, 16 * 32, out))
    assert _expand(B=thin) == L.LORA_ERR_INVALID_ARG                          # slots overlap
    Bz = (L.lora_weight * 2)(L.lora_weight(_base, 16 * 64, 0, 5), L.lora_weight(_base, 16 * 32))
    assert _expand(B=Bz) == L.LORA_ERR_INVALID_ARG                          # reserved != 0


def test_expand_rejections():
    assert _expand(offsets=(0, 32)) == L.LORA_ERR_INVALID_ARG        # windows overlap
    assert _expand(ldy=90) == L.LORA_ERR_INVALID_ARG                 # ldy not a multiple of 8
    assert _expand(ldy=88) == L.LORA_ERR_INVALID_ARG                 # window past ldy
    assert _expand(widths=(64, 30)) == L.LORA_ERR_INVALID_ARG        # width not a multiple of 8
    assert _expand(offsets=(0, 68)) == L.LORA_ERR_INVALID_ARG        # offset not a multiple of 8
    assert _expand(r=20) == L.LORA_ERR_UNSUPPORTED
    assert _expand(r=256) == L.LORA_ERR_UNSUPPORTED
    assert _expand(y=_ptr(2)) == L.LORA_ERR_INVALID_ARG
    thin = (L.lora_weight * 2)(L.lora_weight(_base, 16 * 64), L.lora_weight(_base, 16 * 32 - 8))
    assert _expand(B=thin) == L.LORA_ERR_INVALID_ARG


def test_apply_rejections():
    n = 1
    A, B = _w(1, 64 * 16), _w(1, 16 * 64)
    wd, of = (C.c_int64 * 1)(64), (C.c_int64 * 1)(0)
    args = lambda ws, ws_bytes: (C.byref(_meta()), _ptr(), 64, 64, 1, n, A, B, wd, of, 16,
                                 C.c_float(1.0), None, None, _ptr(), 64, 1, 0, ws, ws_bytes, None)
    big = 1 << 22   # enough for this call: count words, rank buffer, tagged partials
    assert _call("lora_apply", *args(_ptr(), 16)) == L.LORA_ERR_WORKSPACE
    assert _call("lora_apply", *args(_ptr(), L.APPLY_SYNC_BYTES)) == L.LORA_ERR_WORKSPACE
    assert _call("lora_apply", None, *args(_ptr(), big)[1:]) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_apply", *args(None, big)) == L.LORA_ERR_WORKSPACE
    assert _call("lora_apply", *args(_ptr(8), big)) == L.LORA_ERR_WORKSPACE
    bad = _meta()
    bad.tiles = None
    assert _call("lora_apply", C.byref(bad), *args(_ptr(), big)[1:]) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_apply", *args(_ptr(), big)[:15], 63, *args(_ptr(), big)[16:]) == L.LORA_ERR_INVALID_ARG  # ldy


def test_workspace_init_rejections():
    assert _call("lora_apply_workspace_init", None, 1 << 19, None) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_apply_workspace_init", _ptr(8), 1 << 19, None) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_apply_workspace_init", _ptr(), L.APPLY_SYNC_BYTES - 16, None) == L.LORA_ERR_WORKSPACE


def test_moe_meta_rejections():
    m = L.lora_meta()
    sz = C.c_size_t(0)
    assert _call("lora_moe_meta_workspace_bytes", 16, 8, 4, 32, C.byref(sz)) == L.LORA_OK
    assert sz.value >= 4 * 16 * 8
    assert _call("lora_moe_meta_workspace_bytes", 16, 0, 4, 32, C.byref(sz)) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_moe_meta_workspace_bytes", 16, 8, 64, 32, C.byref(sz)) == L.LORA_ERR_UNSUPPORTED
    args = lambda ws_bytes, em=None, topk=8: (_ptr(), 16, topk, _ptr(), 4, 256, 32, em, _ptr(), ws_bytes,
                                             C.byref(m), None)
    assert _call("lora_prepare_moe_meta", *args(16)) == L.LORA_ERR_WORKSPACE
    assert _call("lora_prepare_moe_meta", *args(1 << 15, em=_ptr(2))) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_prepare_moe_meta", *args(1 << 15, topk=0)) == L.LORA_ERR_INVALID_ARG
    bad = _meta()
    bad.x_row_div = 0
    assert _shrink(meta=bad) == L.LORA_ERR_INVALID_ARG


def test_noalloc_rejections():
    """lora_apply_noalloc checks its arguments, and that the call fits the
    library's scratch, before touching a device."""
    A, B = _w(1, 64 * 16), _w(1, 16 * 64)
    wd, of = (C.c_int64 * 1)(64), (C.c_int64 * 1)(0)
    args = lambda meta, r: (C.byref(meta), _ptr(), 64, 64, 1, 1, A, B, wd, of, r, C.c_float(1.0), None, None,
                            _ptr(), 64, 1, 0, None)
    assert _call("lora_apply_noalloc", None, *args(_meta(), 16)[1:]) == L.LORA_ERR_INVALID_ARG
    assert _call("lora_apply_noalloc", *args(_meta(), 12)) == L.LORA_ERR_UNSUPPORTED
    huge = _meta(T=1 << 22, S=4)   # 4 M tokens x 16 ranks of fp32: past the 64 MiB scratch
    assert _call("lora_apply_noalloc", *args(huge, 16)) == L.LORA_ERR_WORKSPACE

