"""The C-ABI library loads without a GPU, exports every function include/attn.h
declares, and rejects bad arguments on the host before anything is enqueued
(no compute call is made here: there is no GPU in this environment)."""
import ctypes
import os
import re

import pytest

import online_softmax_fusion_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, INVALID, UNSUPPORTED = attn.ATTN_OK, attn.ATTN_ERR_INVALID_ARG, attn.ATTN_ERR_UNSUPPORTED

# fake but 16-byte aligned "device" addresses: validation never dereferences them
P1, P2, P3, P4, P5, P6 = (0x10000 * (i + 1) for i in range(6))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:attn|l2norm)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return attn.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd_prefill", "attn_fwd_decode_splitk", "attn_splitk_combine", "attn_bwd", "attn_fwd",
              "l2norm_rows"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_struct_layout_matches(lib):
    assert lib.attn_fwd_args_size() == ctypes.sizeof(attn.AttnFwdArgs) == 272
    assert lib.attn_bwd_args_size() == ctypes.sizeof(attn.AttnBwdArgs) == 416


def test_status_strings(lib):
    for s in range(5):
        assert lib.attn_status_str(s)
    assert lib.attn_status_str(99) == b"unknown status"


def good_args(dtype=attn.ATTN_BF16, D=128):
    a = attn.AttnFwdArgs()
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.D = 2, 8, 2, 64, 96, D
    a.dtype = dtype
    a.causal = 1
    a.q, a.k, a.v = P1, P2, P3
    for name, H, L in (("q_strides", 8, 64), ("k_strides", 2, 96), ("v_strides", 2, 96)):
        setattr(a, name, (ctypes.c_int64 * 3)(H * L * D, L * D, D))
    a.scale = 0.125
    a.o = P4
    a.o_dtype = dtype
    a.o_strides = (ctypes.c_int64 * 3)(8 * 64 * D, 64 * D, D)
    a.lse = P5
    return a


def test_valid_args_pass(lib):
    assert lib.attn_validate_prefill(ctypes.byref(good_args())) == OK
    assert lib.attn_validate_prefill(ctypes.byref(good_args(attn.ATTN_F32, 64))) == OK
    assert lib.attn_validate_decode(ctypes.byref(good_args()), 4, P4, P5, P6) == OK


@pytest.mark.parametrize("mutate,expect", [
    (lambda a: setattr(a, "Hq", 7), INVALID),             # Hq % Hkv != 0
    (lambda a: setattr(a, "Hkv", 0), INVALID),
    (lambda a: setattr(a, "B", -1), INVALID),
    (lambda a: setattr(a, "Lk", -5), INVALID),
    (lambda a: setattr(a, "dtype", 7), INVALID),
    (lambda a: setattr(a, "o_dtype", 3), INVALID),
    (lambda a: setattr(a, "causal", 2), INVALID),
    (lambda a: setattr(a, "scale", float("nan")), INVALID),
    (lambda a: setattr(a, "q", None), INVALID),
    (lambda a: setattr(a, "v", None), INVALID),
    (lambda a: setattr(a, "o", None), INVALID),
    (lambda a: setattr(a, "bias_kind", 5), INVALID),
    (lambda a: setattr(a, "bias_kind", attn.ATTN_BIAS_DENSE), INVALID),   # null bias
    (lambda a: setattr(a, "bias_kind", attn.ATTN_BIAS_ALIBI), INVALID),   # null slopes
    (lambda a: a.k_strides.__setitem__(2, -128), INVALID),
    (lambda a: setattr(a, "softcap", -1.0), INVALID),
    (lambda a: setattr(a, "softcap", float("nan")), INVALID),
    (lambda a: setattr(a, "softcap", float("inf")), INVALID),
    (lambda a: setattr(a, "window", 2), INVALID),
    (lambda a: setattr(a, "D", 96), UNSUPPORTED),
    (lambda a: setattr(a, "D", 256), UNSUPPORTED),
    (lambda a: setattr(a, "q", P1 + 2), UNSUPPORTED),     # misaligned
    (lambda a: a.k_strides.__setitem__(2, 130), UNSUPPORTED),
    (lambda a: setattr(a, "o", P4 + 8), UNSUPPORTED),
])
def test_prefill_rejects(lib, mutate, expect):
    a = good_args()
    mutate(a)
    assert lib.attn_validate_prefill(ctypes.byref(a)) == expect
    # the entry point runs the same check and returns before any HIP call
    assert lib.attn_fwd_prefill(ctypes.byref(a), None) == expect


def test_null_args(lib):
    assert lib.attn_fwd_prefill(None, None) == INVALID
    assert lib.attn_fwd_decode_splitk(None, 1, P4, P5, P6, None) == INVALID


@pytest.mark.parametrize("splits,o_part,expect", [
    (0, P4, INVALID), (-3, P4, INVALID), (65536, P4, INVALID), (4, None, INVALID), (4, P4 + 4, INVALID),
])
def test_decode_rejects(lib, splits, o_part, expect):
    a = good_args()
    assert lib.attn_validate_decode(ctypes.byref(a), splits, o_part, P5, P6) == expect
    assert lib.attn_fwd_decode_splitk(ctypes.byref(a), splits, o_part, P5, P6, None) == expect


def test_combine_rejects(lib):
    st3 = (ctypes.c_int64 * 3)(1024, 128, 128)
    f = lib.attn_splitk_combine
    assert f(P1, P2, P3, 1, 8, 1, 128, 0, P4, attn.ATTN_BF16, st3, P5, None) == INVALID
    assert f(P1, P2, P3, 1, 0, 1, 128, 4, P4, attn.ATTN_BF16, st3, P5, None) == INVALID
    assert f(P1, P2, P3, 1, 8, 1, 96, 4, P4, attn.ATTN_BF16, st3, P5, None) == UNSUPPORTED
    assert f(None, P2, P3, 1, 8, 1, 128, 4, P4, attn.ATTN_BF16, st3, P5, None) == INVALID
    assert f(P1, P2, P3, 1, 8, 1, 128, 4, P4, 9, st3, P5, None) == INVALID
    assert f(P1, P2, P3, 1, 8, 1, 128, 4, P4, attn.ATTN_BF16, None, P5, None) == INVALID


def test_empty_problem_is_ok_without_launch(lib):
    a = good_args()
    a.Lq = 0
    assert lib.attn_fwd_prefill(ctypes.byref(a), None) == OK
    a = good_args()
    a.B = 0
    assert lib.attn_fwd_decode_splitk(ctypes.byref(a), 4, P4, P5, P6, None) == OK


def test_choose_splits(lib):
    # fills one workgroup per compute unit, at least 256 keys per chunk
    assert lib.attn_decode_choose_splits(1, 8, 8, 1, 32768, 256) == 32
    assert lib.attn_decode_choose_splits(16, 32, 8, 1, 32768, 256) == 2
    assert lib.attn_decode_choose_splits(1, 8, 8, 1, 200, 256) == 1
    assert lib.attn_decode_choose_splits(1, 8, 8, 1, 1024, 256) == 4
    assert lib.attn_decode_choose_splits(1, 8, 3, 1, 4096, 256) == 1   # invalid grouping -> 1
    for B, Hkv, Lk in ((1, 1, 10 ** 6), (4, 2, 65536), (64, 8, 4096)):
        S = lib.attn_decode_choose_splits(B, Hkv, Hkv, 1, Lk, 256)
        assert 1 <= S <= max(1, Lk // 256)


def test_partial_bytes(lib):
    # C4: 16 * 32 rows, 32 chunks, D = 128: (128 + 2) * 4 bytes per (row, chunk)
    assert lib.attn_decode_partial_bytes(16, 32, 1, 128, 32) == 16 * 32 * 32 * 130 * 4


def test_chunk_length():
    assert attn.chunk_length(32768, 32) == 1024
    assert attn.chunk_length(1000, 3) == 352
    assert attn.chunk_length(100, 10) == 32
    assert attn.chunk_length(0, 4) == 32


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------
P7, P8, P9, P10 = (0x10000 * (i + 7) for i in range(4))


def good_bwd_args(grad_dtype=attn.ATTN_F32, D=128):
    b = attn.AttnBwdArgs()
    b.fwd = good_args(attn.ATTN_BF16, D)
    b.dout = P6
    b.dout_strides = (ctypes.c_int64 * 3)(8 * 64 * D, 64 * D, D)
    b.grad_dtype = grad_dtype
    b.dq, b.dk, b.dv = P7, P8, P9
    b.dq_strides = (ctypes.c_int64 * 3)(8 * 64 * D, 64 * D, D)
    b.dk_strides = (ctypes.c_int64 * 3)(2 * 96 * D, 96 * D, D)
    b.dv_strides = (ctypes.c_int64 * 3)(2 * 96 * D, 96 * D, D)
    b.workspace = P10
    return b


def test_bwd_valid_args_pass(lib):
    assert lib.attn_validate_bwd(ctypes.byref(good_bwd_args())) == OK
    assert lib.attn_validate_bwd(ctypes.byref(good_bwd_args(attn.ATTN_BF16, 64))) == OK


@pytest.mark.parametrize("mutate,expect", [
    (lambda b: setattr(b.fwd, "lse", None), INVALID),        # the saved LSE is required
    (lambda b: setattr(b.fwd, "o", None), INVALID),
    (lambda b: setattr(b, "dout", None), INVALID),
    (lambda b: setattr(b, "dq", None), INVALID),
    (lambda b: setattr(b, "dk", None), INVALID),
    (lambda b: setattr(b, "dv", None), INVALID),
    (lambda b: setattr(b, "workspace", None), INVALID),
    (lambda b: setattr(b, "workspace", P10 + 4), INVALID),
    (lambda b: setattr(b, "grad_dtype", 5), INVALID),
    (lambda b: setattr(b, "reserved", 1), INVALID),
    (lambda b: b.dq_strides.__setitem__(1, -1), INVALID),
    (lambda b: setattr(b.fwd, "causal", 3), INVALID),
    (lambda b: setattr(b.fwd, "softcap", -2.0), INVALID),
    (lambda b: setattr(b.fwd, "dtype", attn.ATTN_F32), UNSUPPORTED),   # fp32 inputs: forward only
    (lambda b: setattr(b.fwd, "D", 96), UNSUPPORTED),
    (lambda b: setattr(b, "dout", P6 + 2), UNSUPPORTED),
    (lambda b: setattr(b, "dk", P8 + 8), UNSUPPORTED),
    (lambda b: b.dv_strides.__setitem__(2, 130), UNSUPPORTED),
])
def test_bwd_rejects(lib, mutate, expect):
    b = good_bwd_args()
    mutate(b)
    assert lib.attn_validate_bwd(ctypes.byref(b)) == expect
    assert lib.attn_bwd(ctypes.byref(b), None) == expect


def test_bwd_null_and_empty(lib):
    assert lib.attn_bwd(None, None) == INVALID
    b = good_bwd_args()
    b.fwd.B = 0
    assert lib.attn_bwd(ctypes.byref(b), None) == OK


def test_bwd_workspace_bytes(lib):
    # two fp32 arrays of B*Hq*Lq values, each rounded up to 16 bytes
    assert lib.attn_bwd_workspace_bytes(2, 3, 5) == 2 * 32 * 4
    assert lib.attn_bwd_workspace_bytes(1, 1, 4) == 32
    assert lib.attn_bwd_workspace_bytes(0, 8, 8) == 0


# ----------------------------------------------------------------------------
# row L2 norm
# ----------------------------------------------------------------------------
def good_l2(H=4096, dtype=attn.ATTN_BF16):
    a = attn.L2NormArgs()
    a.rows, a.H = 10, H
    a.x_dtype = a.y_dtype = dtype
    a.x, a.x_stride = P1, H
    a.y, a.y_stride = P2, H
    a.norm = P3
    return a


def test_l2norm_struct_and_limits(lib):
    assert lib.l2norm_args_size() == ctypes.sizeof(attn.L2NormArgs) == 64
    assert lib.l2norm_max_onepass(attn.ATTN_BF16) == 8192
    assert lib.l2norm_max_onepass(attn.ATTN_F32) == 4096
    assert lib.l2norm_validate(ctypes.byref(good_l2()), 1) == OK
    assert lib.l2norm_validate(ctypes.byref(good_l2(100000)), 7) == OK


@pytest.mark.parametrize("mutate,splits,expect", [
    (lambda a: setattr(a, "rows", -1), 1, INVALID),
    (lambda a: setattr(a, "x_dtype", 5), 1, INVALID),
    (lambda a: setattr(a, "x", None), 1, INVALID),
    (lambda a: setattr(a, "x_stride", 100), 1, INVALID),        # shorter than a row
    (lambda a: (setattr(a, "y", None), setattr(a, "norm", None)), 1, INVALID),   # nothing to write
    (lambda a: setattr(a, "norm", P3 + 2), 1, INVALID),
    (lambda a: None, 0, INVALID),
    (lambda a: setattr(a, "H", 4100), 1, UNSUPPORTED),          # not a multiple of 8 bf16
    (lambda a: setattr(a, "x", P1 + 8), 1, UNSUPPORTED),
    (lambda a: setattr(a, "y_stride", 4100), 1, UNSUPPORTED),
    (lambda a: setattr(a, "H", 8200), 1, UNSUPPORTED),          # too long for one pass
])
def test_l2norm_rejects(lib, mutate, splits, expect):
    a = good_l2()
    a.x_stride = a.y_stride = 8200
    mutate(a)
    assert lib.l2norm_validate(ctypes.byref(a), splits) == expect
    assert lib.l2norm_rows(ctypes.byref(a), splits, None, 0, None) == expect


def test_l2norm_split_workspace_checked_first(lib):
    a = good_l2(100000)
    a.x_stride = a.y_stride = 100000
    assert lib.l2norm_workspace_bytes(10, 7) == 10 * 7 * 8
    assert lib.l2norm_rows(ctypes.byref(a), 7, None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert lib.l2norm_rows(ctypes.byref(a), 7, P4, 10 * 7 * 8 - 1, None) == attn.ATTN_ERR_WORKSPACE


def test_l2norm_choose_splits(lib):
    f = lib.l2norm_choose_splits
    assert f(32768, 4096, attn.ATTN_BF16, 256) == 1          # fits one pass
    assert f(8, 8192, attn.ATTN_BF16, 256) == 1
    assert f(8, 8200, attn.ATTN_BF16, 256) == 4               # 16400 bytes: at least 4096 per chunk
    assert f(8, 4194304, attn.ATTN_F32, 256) == 128           # four workgroups per CU
    assert f(10000, 1 << 20, attn.ATTN_BF16, 256) == 2        # enough rows already: the minimum split
    assert f(0, 1 << 20, attn.ATTN_BF16, 256) == 1
