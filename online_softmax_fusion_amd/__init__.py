"""Python binding of the MI355X fused attention library (forward and backward).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libattn_mi355x.so`` behind the C ABI of ``include/attn.h``.
PyTorch supplies device memory and the current HIP stream.  There is no CPU
or PyTorch fallback: if the library is missing, loading fails loudly.

Entry points (same names as the C ABI):
    attn_fwd_prefill(q, k, v, ...)             -> (o, lse)
    attn_fwd_decode_splitk(q, k, v, splits, ...) -> (o_part, m_part, l_part)
    attn_splitk_combine(o_part, m_part, l_part, ...) -> (o, lse)
    attn_fwd(q, k, v, ...)                     -> (o, lse)   (planned: prefill or split-K)
    attn_fwd_choose_plan(q, k, v, ...)         -> AttnFwdPlan
    attn_bwd(q, k, v, o, lse, dout, ...)       -> (dq, dk, dv)
    l2norm_rows(x, ...)                        -> (y, norm)  (include/l2norm.h)
and the conveniences ``prefill`` (= attn_fwd_prefill) and ``decode`` (split-K
local step followed by the combine on the same stream).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "AttnError", "load_library", "library_path", "attn_fwd_prefill", "attn_fwd_decode_splitk",
    "attn_splitk_combine", "attn_decode_choose_splits", "attn_decode_partial_bytes",
    "attn_device_cu_count", "attn_device_xcd_count", "prefill", "decode", "chunk_length", "AttnFwdArgs", "AttnBwdArgs", "attn_bwd",
    "attn_bwd_workspace_bytes", "attn_fwd", "attn_fwd_choose_plan", "AttnFwdPlan", "ATTN_PLAN_PREFILL",
    "ATTN_PLAN_SPLITK", "ATTN_PLAN_PREFILL_SPLIT", "attn_fwd_prefill_splitk", "attn_prefill_choose_splits", "L2NormArgs", "l2norm_rows", "l2norm_choose_splits", "l2norm_workspace_bytes",
    "l2norm_max_onepass",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn_mi355x.so")
_LIB = None

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = 0, 1, 2, 3, 4
ATTN_F32, ATTN_BF16 = 0, 1
ATTN_BIAS_NONE, ATTN_BIAS_DENSE, ATTN_BIAS_ALIBI = 0, 1, 2
ATTN_PLAN_PREFILL, ATTN_PLAN_SPLITK, ATTN_PLAN_PREFILL_SPLIT = 0, 1, 2

_I64x3 = ctypes.c_int64 * 3
_I64x4 = ctypes.c_int64 * 4


class AttnFwdArgs(ctypes.Structure):
    """Mirror of ``attn_fwd_args`` in include/attn.h (field order and types)."""
    _fields_ = [
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("Lq", ctypes.c_int64), ("Lk", ctypes.c_int64), ("D", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_strides", _I64x3), ("k_strides", _I64x3), ("v_strides", _I64x3),
        ("scale", ctypes.c_float), ("bias_kind", ctypes.c_int32),
        ("bias", ctypes.c_void_p), ("bias_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
        ("bias_strides", _I64x4), ("alibi_slopes", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("o_strides", _I64x3), ("lse", ctypes.c_void_p),
        ("softcap", ctypes.c_float), ("window", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
    ]


class AttnFwdPlan(ctypes.Structure):
    """Mirror of ``attn_fwd_plan`` in include/attn.h."""
    _fields_ = [("method", ctypes.c_int32), ("num_splits", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


class AttnBwdArgs(ctypes.Structure):
    """Mirror of ``attn_bwd_args`` in include/attn.h."""
    _fields_ = [
        ("fwd", AttnFwdArgs),
        ("dout", ctypes.c_void_p), ("dout_strides", _I64x3),
        ("grad_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("dq", ctypes.c_void_p), ("dq_strides", _I64x3),
        ("dk", ctypes.c_void_p), ("dk_strides", _I64x3),
        ("dv", ctypes.c_void_p), ("dv_strides", _I64x3),
        ("workspace", ctypes.c_void_p),
    ]


class L2NormArgs(ctypes.Structure):
    """Mirror of ``l2norm_args`` in include/l2norm.h."""
    _fields_ = [
        ("rows", ctypes.c_int64), ("H", ctypes.c_int64),
        ("x_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("x_stride", ctypes.c_int64),
        ("y", ctypes.c_void_p), ("y_stride", ctypes.c_int64),
        ("norm", ctypes.c_void_p),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = load_library()
        msg = lib.attn_status_str(status).decode()
        super().__init__("%s failed: %s (status %d)" % (what, msg, status))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libattn_mi355x.so; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libattn_mi355x.so is not built (run __graft_entry__.build() or "
                          "python online_softmax_fusion_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(AttnFwdArgs)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.attn_fwd_prefill.argtypes = [P, vp]
    lib.attn_fwd_prefill.restype = ctypes.c_int
    lib.attn_fwd_decode_splitk.argtypes = [P, i32, vp, vp, vp, vp]
    lib.attn_fwd_decode_splitk.restype = ctypes.c_int
    lib.attn_fwd_prefill_splitk.argtypes = [P, i32, vp, vp, vp, vp]
    lib.attn_fwd_prefill_splitk.restype = ctypes.c_int
    lib.attn_prefill_choose_splits.argtypes = [i64, i64, i64, i64, i32]
    lib.attn_prefill_choose_splits.restype = i32
    lib.attn_splitk_combine.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, vp, i32,
                                        ctypes.POINTER(ctypes.c_int64), vp, vp]
    lib.attn_splitk_combine.restype = ctypes.c_int
    lib.attn_decode_choose_splits.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.attn_decode_choose_splits.restype = i32
    lib.attn_decode_partial_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.attn_decode_partial_bytes.restype = ctypes.c_size_t
    lib.attn_device_cu_count.argtypes = [i32]
    lib.attn_device_cu_count.restype = i32
    lib.attn_device_xcd_count.argtypes = [i32]
    lib.attn_device_xcd_count.restype = i32
    lib.attn_validate_prefill.argtypes = [P]
    lib.attn_validate_prefill.restype = ctypes.c_int
    lib.attn_validate_decode.argtypes = [P, i32, vp, vp, vp]
    lib.attn_validate_decode.restype = ctypes.c_int
    lib.attn_status_str.argtypes = [ctypes.c_int]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_fwd_args_size.argtypes = []
    lib.attn_fwd_args_size.restype = ctypes.c_size_t
    lib.attn_fwd_choose_plan.argtypes = [P, i32, ctypes.POINTER(AttnFwdPlan)]
    lib.attn_fwd_choose_plan.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [P, vp, ctypes.c_size_t, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_noalloc.argtypes = [P, vp]
    lib.attn_fwd_noalloc.restype = ctypes.c_int
    PB = ctypes.POINTER(AttnBwdArgs)
    lib.attn_bwd.argtypes = [PB, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_validate_bwd.argtypes = [PB]
    lib.attn_validate_bwd.restype = ctypes.c_int
    lib.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_args_size.argtypes = []
    lib.attn_bwd_args_size.restype = ctypes.c_size_t
    PL = ctypes.POINTER(L2NormArgs)
    lib.l2norm_rows.argtypes = [PL, i32, vp, ctypes.c_size_t, vp]
    lib.l2norm_rows.restype = ctypes.c_int
    lib.l2norm_validate.argtypes = [PL, i32]
    lib.l2norm_validate.restype = ctypes.c_int
    lib.l2norm_choose_splits.argtypes = [i64, i64, i32, i32]
    lib.l2norm_choose_splits.restype = i32
    lib.l2norm_max_onepass.argtypes = [i32]
    lib.l2norm_max_onepass.restype = i64
    lib.l2norm_workspace_bytes.argtypes = [i64, i32]
    lib.l2norm_workspace_bytes.restype = ctypes.c_size_t
    lib.l2norm_args_size.argtypes = []
    lib.l2norm_args_size.restype = ctypes.c_size_t
    if lib.l2norm_args_size() != ctypes.sizeof(L2NormArgs):
        raise ImportError("l2norm_args layout mismatch between include/l2norm.h and the binding")
    if lib.attn_fwd_args_size() != ctypes.sizeof(AttnFwdArgs):
        raise ImportError("attn_fwd_args layout mismatch between include/attn.h and the binding")
    if lib.attn_bwd_args_size() != ctypes.sizeof(AttnBwdArgs):
        raise ImportError("attn_bwd_args layout mismatch between include/attn.h and the binding")
    _LIB = lib
    return lib


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return ATTN_BF16
    if t == torch.float32:
        return ATTN_F32
    raise TypeError("only bfloat16 and float32 tensors are supported, got %s" % t)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check_4d(name: str, t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError("%s must be 4-D [B, H, L, D], got shape %s" % (name, tuple(t.shape)))
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("%s must have a contiguous last dimension" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)


def _on(dev: torch.device, name: str, t: Optional[torch.Tensor]):
    """Every buffer of one call lives on the device the kernels run on."""
    if t is not None and (not t.is_cuda or t.device != dev):
        raise ValueError("%s must be on %s, got %s" % (name, dev, t.device))


def _check_out(name: str, t: torch.Tensor, shape, dev: torch.device):
    _check_4d(name, t)
    _on(dev, name, t)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_lse(lse: torch.Tensor, n: int, dev: torch.device):
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != n:
        raise ValueError("lse must be a contiguous fp32 tensor of %d elements" % n)
    _on(dev, "lse", lse)


def _strides3(t: torch.Tensor):
    return _I64x3(*[int(x) for x in t.stride()[:3]])


def _make_args(q, k, v, scale, causal, bias, alibi_slopes, o=None, lse=None, softcap=0.0,
               window=None) -> AttnFwdArgs:
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_4d(name, t)
        _on(q.device, name, t)
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k and v must share one dtype")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if tuple(v.shape) != (Bk, Hkv, Lk, Dk) or Bk != B or Dk != D:
        raise ValueError("shape mismatch: q %s, k %s, v %s" % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    a = AttnFwdArgs()
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.D = B, Hq, Hkv, Lq, Lk, D
    a.dtype = _dtype_code(q.dtype)
    a.causal = 1 if causal else 0
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.q_strides, a.k_strides, a.v_strides = _strides3(q), _strides3(k), _strides3(v)
    a.scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
    a.bias_kind = ATTN_BIAS_NONE
    a.bias_dtype = ATTN_F32
    if bias is not None and alibi_slopes is not None:
        raise ValueError("give either a dense bias or ALiBi slopes, not both")
    if bias is not None:
        _on(q.device, "bias", bias)
        bb = bias
        while bb.dim() < 4:
            bb = bb.unsqueeze(0)
        bb = bb.expand(B, Hq, Lq, Lk)
        a.bias_kind = ATTN_BIAS_DENSE
        a.bias = bb.data_ptr()
        a.bias_dtype = _dtype_code(bb.dtype)
        a.bias_strides = _I64x4(*[int(x) for x in bb.stride()])
    elif alibi_slopes is not None:
        _on(q.device, "alibi_slopes", alibi_slopes)
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != Hq:
            raise ValueError("alibi_slopes must be a GPU fp32 tensor with one slope per query head")
        slopes = alibi_slopes.contiguous()
        a._keep = (slopes,)   # a contiguous copy must outlive the launch that reads it
        a.bias_kind = ATTN_BIAS_ALIBI
        a.alibi_slopes = slopes.data_ptr()
    if o is not None:
        _on(q.device, "out", o)
        a.o = _ptr(o)
        a.o_dtype = _dtype_code(o.dtype)
        a.o_strides = _strides3(o)
    else:
        a.o_dtype = a.dtype
    a.lse = _ptr(lse)
    a.softcap = float(softcap or 0.0)
    if window is not None:
        a.window = 1
        a.window_left, a.window_right = int(window[0]), int(window[1])
    return a


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
def attn_fwd_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                     causal: bool = False, *, bias: Optional[torch.Tensor] = None,
                     alibi_slopes: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     out_dtype: Optional[torch.dtype] = None, lse: Optional[torch.Tensor] = None,
                     return_lse: bool = True, softcap: float = 0.0,
                     window: Optional[Tuple[int, int]] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused attention forward (rolling update).  q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D].

    Returns (O [B,Hq,Lq,D], LSE [B,Hq,Lq] fp32 or None).  ``bias`` broadcasts to
    [B,Hq,Lq,Lk]; ``alibi_slopes`` is an fp32 [Hq] tensor; ``softcap`` > 0 caps
    the scaled score; ``window`` = (left, right) keys around each query's
    position (negative = unbounded).
    """
    lib = load_library()
    _check_4d("q", q)
    B, Hq, Lq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=out_dtype or q.dtype, device=q.device)
    else:
        _check_out("out", out, (B, Hq, Lq, D), q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_lse(lse, B * Hq * Lq, q.device)
    a = _make_args(q, k, v, scale, causal, bias, alibi_slopes, out, lse, softcap, window)
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_prefill(ctypes.byref(a), _stream(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_prefill")
    return out, lse


prefill = attn_fwd_prefill


def chunk_length(Lk: int, num_splits: int) -> int:
    """Keys per split-K chunk: 32 * ceil(Lk / (32 * num_splits)) (include/attn.h)."""
    per = -(-Lk // (32 * num_splits))
    return 32 * max(per, 1)


def attn_fwd_decode_splitk(q, k, v, num_splits: int, scale: Optional[float] = None, causal: bool = False, *,
                           bias=None, alibi_slopes=None, o_part=None, m_part=None, l_part=None,
                           softcap: float = 0.0, window: Optional[Tuple[int, int]] = None):
    """Split-K local step: partials (o [B,Hq,Lq,S,D], m [B,Hq,Lq,S], l [B,Hq,Lq,S]) in fp32."""
    lib = load_library()
    _check_4d("q", q)
    B, Hq, Lq, D = q.shape
    S = int(num_splits)
    dev = q.device
    if o_part is None:
        o_part = torch.empty((B, Hq, Lq, S, D), dtype=torch.float32, device=dev)
    if m_part is None:
        m_part = torch.empty((B, Hq, Lq, S), dtype=torch.float32, device=dev)
    if l_part is None:
        l_part = torch.empty((B, Hq, Lq, S), dtype=torch.float32, device=dev)
    for name, t, n in (("o_part", o_part, B * Hq * Lq * S * D), ("m_part", m_part, B * Hq * Lq * S),
                       ("l_part", l_part, B * Hq * Lq * S)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError("%s must be a contiguous GPU fp32 tensor of %d elements" % (name, n))
        _on(dev, name, t)
    a = _make_args(q, k, v, scale, causal, bias, alibi_slopes, softcap=softcap, window=window)
    with torch.cuda.device(dev):
        st = lib.attn_fwd_decode_splitk(ctypes.byref(a), S, _ptr(o_part), _ptr(m_part), _ptr(l_part),
                                        _stream(dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_decode_splitk")
    return o_part, m_part, l_part


def prefill_chunk_length(Lk: int, num_splits: int) -> int:
    """Keys per chunk of the split prefill: 64 * ceil(Lk / (64 * num_splits)) (include/attn.h)."""
    per = -(-Lk // (64 * num_splits))
    return 64 * max(per, 1)


def attn_fwd_prefill_splitk(q, k, v, num_splits: int, scale: Optional[float] = None, causal: bool = False, *,
                            bias=None, alibi_slopes=None, o_part=None, m_part=None, l_part=None,
                            softcap: float = 0.0, window: Optional[Tuple[int, int]] = None):
    """Prefill over key chunks: partials (o [B,Hq,Lq,S,D], m [B,Hq,Lq,S], l [B,Hq,Lq,S]) in fp32,
    in the layout of attn_fwd_decode_splitk, for attn_splitk_combine."""
    lib = load_library()
    _check_4d("q", q)
    B, Hq, Lq, D = q.shape
    S = int(num_splits)
    dev = q.device
    if o_part is None:
        o_part = torch.empty((B, Hq, Lq, S, D), dtype=torch.float32, device=dev)
    if m_part is None:
        m_part = torch.empty((B, Hq, Lq, S), dtype=torch.float32, device=dev)
    if l_part is None:
        l_part = torch.empty((B, Hq, Lq, S), dtype=torch.float32, device=dev)
    for name, t, n in (("o_part", o_part, B * Hq * Lq * S * D), ("m_part", m_part, B * Hq * Lq * S),
                       ("l_part", l_part, B * Hq * Lq * S)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError("%s must be a contiguous GPU fp32 tensor of %d elements" % (name, n))
        _on(dev, name, t)
    a = _make_args(q, k, v, scale, causal, bias, alibi_slopes, softcap=softcap, window=window)
    with torch.cuda.device(dev):
        st = lib.attn_fwd_prefill_splitk(ctypes.byref(a), S, _ptr(o_part), _ptr(m_part), _ptr(l_part),
                                         _stream(dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_prefill_splitk")
    return o_part, m_part, l_part


def attn_prefill_choose_splits(B: int, Hq: int, Lq: int, Lk: int, cu_count: int = 0) -> int:
    return int(load_library().attn_prefill_choose_splits(B, Hq, Lq, Lk, cu_count))


def attn_splitk_combine(o_part, m_part, l_part, *, out=None, out_dtype=torch.bfloat16, lse=None,
                        return_lse: bool = True):
    """Split-K global step: (O [B,Hq,Lq,D], LSE [B,Hq,Lq]) from the partials."""
    lib = load_library()
    if o_part.dim() != 5:
        raise ValueError("o_part must be [B, Hq, Lq, S, D]")
    B, Hq, Lq, S, D = o_part.shape
    dev = o_part.device
    for name, t in (("o_part", o_part), ("m_part", m_part), ("l_part", l_part)):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous GPU fp32 tensor" % name)
        _on(dev, name, t)
    if tuple(m_part.shape) != (B, Hq, Lq, S) or tuple(l_part.shape) != (B, Hq, Lq, S):
        raise ValueError("m_part and l_part must be [B, Hq, Lq, S]")
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=out_dtype, device=dev)
    else:
        _check_out("out", out, (B, Hq, Lq, D), dev)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_lse(lse, B * Hq * Lq, dev)
    with torch.cuda.device(dev):
        st = lib.attn_splitk_combine(_ptr(o_part), _ptr(m_part), _ptr(l_part), B, Hq, Lq, D, S, _ptr(out),
                                     _dtype_code(out.dtype), _strides3(out), _ptr(lse), _stream(dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_splitk_combine")
    return out, lse


def attn_decode_choose_splits(B: int, Hq: int, Hkv: int, Lq: int, Lk: int, cu_count: int = 0) -> int:
    return int(load_library().attn_decode_choose_splits(B, Hq, Hkv, Lq, Lk, cu_count))


def attn_decode_partial_bytes(B: int, Hq: int, Lq: int, D: int, num_splits: int) -> int:
    return int(load_library().attn_decode_partial_bytes(B, Hq, Lq, D, num_splits))


def attn_device_cu_count(device: int = 0) -> int:
    return int(load_library().attn_device_cu_count(device))


def attn_device_xcd_count(device: int = 0) -> int:
    return int(load_library().attn_device_xcd_count(device))


def decode(q, k, v, num_splits: Optional[int] = None, scale: Optional[float] = None, causal: bool = False, *,
           bias=None, alibi_slopes=None, out=None, out_dtype=None, workspace=None, return_lse: bool = True,
           softcap: float = 0.0, window: Optional[Tuple[int, int]] = None):
    """Split-K decode: local step then combine, both enqueued on the current stream.

    ``workspace`` may be a tuple (o_part, m_part, l_part) to reuse.
    """
    B, Hq, Lq, D = q.shape
    if num_splits is None:
        cu = attn_device_cu_count(q.device.index or 0)
        num_splits = attn_decode_choose_splits(B, Hq, k.shape[1], Lq, k.shape[2], cu)
    o_part = m_part = l_part = None
    if workspace is not None:
        o_part, m_part, l_part = workspace
    o_part, m_part, l_part = attn_fwd_decode_splitk(q, k, v, num_splits, scale, causal, bias=bias,
                                                    alibi_slopes=alibi_slopes, o_part=o_part,
                                                    m_part=m_part, l_part=l_part, softcap=softcap,
                                                    window=window)
    return attn_splitk_combine(o_part, m_part, l_part, out=out, out_dtype=out_dtype or q.dtype,
                               return_lse=return_lse)


def attn_bwd_workspace_bytes(B: int, Hq: int, Lq: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, Hq, Lq))


def attn_bwd(q, k, v, o, lse, dout, scale: Optional[float] = None, causal: bool = False, *, bias=None,
             alibi_slopes=None, softcap: float = 0.0, window: Optional[Tuple[int, int]] = None,
             grad_dtype: Optional[torch.dtype] = None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dQ [B,Hq,Lq,D], dK [B,Hkv,Lk,D], dV [B,Hkv,Lk,D]) of attention
    for the output gradient ``dout``.  ``o`` and ``lse`` are the forward's
    outputs for the same arguments; the other arguments are as for
    ``attn_fwd_prefill``.  ``workspace`` may be a GPU byte tensor of at least
    ``attn_bwd_workspace_bytes(B, Hq, Lq)`` bytes to reuse."""
    lib = load_library()
    _check_4d("q", q)
    _check_4d("k", k)
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    dev = q.device
    for name, t in (("o", o), ("dout", dout)):
        _check_out(name, t, (B, Hq, Lq, D), dev)
    if dout.dtype != q.dtype:
        raise TypeError("dout must have the dtype of q")
    _check_lse(lse, B * Hq * Lq, dev)
    gdt = grad_dtype or q.dtype
    if dq is None:
        dq = torch.empty((B, Hq, Lq, D), dtype=gdt, device=dev)
    if dk is None:
        dk = torch.empty((B, Hkv, Lk, D), dtype=gdt, device=dev)
    if dv is None:
        dv = torch.empty((B, Hkv, Lk, D), dtype=gdt, device=dev)
    for name, t, shape in (("dq", dq, (B, Hq, Lq, D)), ("dk", dk, (B, Hkv, Lk, D)), ("dv", dv, (B, Hkv, Lk, D))):
        _check_out(name, t, shape, dev)
        if t.dtype != gdt:
            raise ValueError("%s must be %s of dtype %s" % (name, shape, gdt))
    need = attn_bwd_workspace_bytes(B, Hq, Lq)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace must be a GPU tensor of at least %d bytes" % need)
    _on(dev, "workspace", workspace)
    a = AttnBwdArgs()
    fa = _make_args(q, k, v, scale, causal, bias, alibi_slopes, o, lse, softcap, window)
    a.fwd = fa   # copies the fields; fa keeps any temporary they point to alive until the launch
    a.dout, a.dout_strides = _ptr(dout), _strides3(dout)
    a.grad_dtype = _dtype_code(gdt)
    a.dq, a.dq_strides = _ptr(dq), _strides3(dq)
    a.dk, a.dk_strides = _ptr(dk), _strides3(dk)
    a.dv, a.dv_strides = _ptr(dv), _strides3(dv)
    a.workspace = _ptr(workspace)
    with torch.cuda.device(dev):
        st = lib.attn_bwd(ctypes.byref(a), _stream(dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def attn_fwd_choose_plan(q, k, v, scale: Optional[float] = None, causal: bool = False, *, bias=None,
                         alibi_slopes=None, softcap: float = 0.0, window: Optional[Tuple[int, int]] = None,
                         cu_count: int = 0, out_dtype: Optional[torch.dtype] = None) -> AttnFwdPlan:
    """The plan (prefill or split-K with its split count and workspace size)
    attn_fwd would run for these arguments on a device with ``cu_count``
    compute units (0: the count of the device q is on)."""
    lib = load_library()
    if cu_count <= 0:
        cu_count = attn_device_cu_count(q.device.index or 0)
    out = torch.empty((1,), dtype=out_dtype or q.dtype, device=q.device)
    a = _make_args(q, k, v, scale, causal, bias, alibi_slopes, None, None, softcap, window)
    a.o, a.o_dtype = out.data_ptr(), _dtype_code(out.dtype)
    B, Hq, Lq, D = q.shape
    a.o_strides = _I64x3(Hq * Lq * D, Lq * D, D)
    plan = AttnFwdPlan()
    st = lib.attn_fwd_choose_plan(ctypes.byref(a), int(cu_count), ctypes.byref(plan))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_choose_plan")
    return plan


def attn_fwd(q, k, v, scale: Optional[float] = None, causal: bool = False, *, bias=None, alibi_slopes=None,
             out=None, out_dtype: Optional[torch.dtype] = None, lse=None, return_lse: bool = True,
             softcap: float = 0.0, window: Optional[Tuple[int, int]] = None, workspace=None):
    """Forward with the automatically chosen parallel dimensions (prefill,
    grouped split-K plus combine, or prefill over key chunks plus combine).  Same arguments and results as
    ``attn_fwd_prefill``; ``workspace`` may be a GPU byte tensor to reuse (a
    new one of the plan's size is allocated otherwise)."""
    lib = load_library()
    _check_4d("q", q)
    B, Hq, Lq, D = q.shape
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=out_dtype or q.dtype, device=q.device)
    else:
        _check_out("out", out, (B, Hq, Lq, D), q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_lse(lse, B * Hq * Lq, q.device)
    a = _make_args(q, k, v, scale, causal, bias, alibi_slopes, out, lse, softcap, window)
    plan = AttnFwdPlan()
    st = lib.attn_fwd_choose_plan(ctypes.byref(a), attn_device_cu_count(q.device.index or 0), ctypes.byref(plan))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_choose_plan")
    if workspace is None and plan.workspace_bytes > 0:
        workspace = torch.empty((plan.workspace_bytes,), dtype=torch.uint8, device=q.device)
    _on(q.device, "workspace", workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib.attn_fwd(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")
    return out, lse


def attn_fwd_noalloc(q, k, v, scale: Optional[float] = None, causal: bool = False, *, bias=None,
                     alibi_slopes=None, out=None, lse=None, softcap: float = 0.0,
                     window: Optional[Tuple[int, int]] = None):
    """``attn_fwd`` without a workspace: the split plans keep their partials in
    the library's fixed per-device array.  ``out`` (and ``lse``, if wanted) must be
    given, so that the call itself allocates nothing; returns them."""
    lib = load_library()
    _check_4d("q", q)
    B, Hq, Lq, D = q.shape
    if out is None:
        raise ValueError("attn_fwd_noalloc: out must be given")
    _check_out("out", out, (B, Hq, Lq, D), q.device)
    if lse is not None:
        _check_lse(lse, B * Hq * Lq, q.device)
    a = _make_args(q, k, v, scale, causal, bias, alibi_slopes, out, lse, softcap, window)
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_noalloc(ctypes.byref(a), _stream(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_noalloc")
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20


def l2norm_max_onepass(dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load_library().l2norm_max_onepass(_dtype_code(dtype)))


def l2norm_choose_splits(rows: int, H: int, dtype: torch.dtype = torch.bfloat16, cu_count: int = 0) -> int:
    return int(load_library().l2norm_choose_splits(rows, H, _dtype_code(dtype), cu_count))


def l2norm_workspace_bytes(rows: int, num_splits: int) -> int:
    return int(load_library().l2norm_workspace_bytes(rows, num_splits))


def l2norm_rows(x, *, out=None, out_dtype: Optional[torch.dtype] = None, norm=None, return_y: bool = True,
                num_splits: Optional[int] = None, workspace=None):
    """Row L2 norm of a 2-D GPU tensor x [rows, H] (bf16 or fp32, unit stride
    along H): returns (y = x / norm or None, norm [rows] fp32).  num_splits
    None picks one pass or split-K (l2norm_choose_splits)."""
    lib = load_library()
    if x.dim() != 2 or not x.is_cuda or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be a 2-D GPU tensor with unit stride along rows")
    rows, H = x.shape
    if num_splits is None:
        num_splits = l2norm_choose_splits(rows, H, x.dtype, attn_device_cu_count(x.device.index or 0))
    if out is None and return_y:
        out = torch.empty((rows, H), dtype=out_dtype or x.dtype, device=x.device)
    if norm is None:
        norm = torch.empty((rows,), dtype=torch.float32, device=x.device)
    elif norm.dtype != torch.float32 or not norm.is_contiguous() or norm.numel() != rows:
        raise ValueError("norm must be a contiguous fp32 tensor of %d elements" % rows)
    _on(x.device, "norm", norm)
    need = l2norm_workspace_bytes(rows, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    _on(x.device, "workspace", workspace)
    a = L2NormArgs()
    a.rows, a.H = rows, H
    a.x_dtype = _dtype_code(x.dtype)
    a.x, a.x_stride = x.data_ptr(), int(x.stride(0)) if rows > 0 else H
    if out is not None:
        if out.shape != x.shape or (H > 1 and out.stride(1) != 1):
            raise ValueError("out must be [rows, H] with unit stride along rows")
        _on(x.device, "out", out)
        a.y, a.y_stride, a.y_dtype = out.data_ptr(), int(out.stride(0)) if rows > 0 else H, _dtype_code(out.dtype)
    a.norm = norm.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        st = lib.l2norm_rows(ctypes.byref(a), int(num_splits), _ptr(workspace), ws_bytes, _stream(x.device))
    if st != ATTN_OK:
        raise AttnError(st, "l2norm_rows")
    return out, norm
