"""fp64 CPU oracle for fused attention (forward, split-K combine, gradients)
and for the row-wise L2 norm.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP path (``online_softmax_fusion_amd``) and imports nothing from it.

The arithmetic lives in ``attn_oracle.c`` (plain C, double precision): the
definition of the attention chain with a two-pass stable softmax, as written in
"Neptune论文浅读" section 2 and in the ``softmax_standard`` listing of the CANN
FlashAttention post.  This module only marshals numpy/torch arrays into it.

Every function here is pinned by ``tests/test_oracle_pins.py`` to values fixed
by the pages and by mathematics (closed forms, invariants, a library softmax on
the full score matrix); see the header of that file for the list.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_LIB = None

BIAS_NONE, BIAS_DENSE, BIAS_ALIBI = 0, 1, 2


def load():
    """Load the compiled oracle; compile it first only when nothing is built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_build.LIB):
        _build.build()
    _LIB = load_path(_build.LIB)
    return _LIB


def load_path(path: str):
    """Load an oracle library from ``path`` (the tests load deliberately broken
    copies this way to show that the pins reject them)."""
    lib = ctypes.CDLL(path)
    i64, dbl, vp = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.oracle_attention.argtypes = [i64, i64, i64, i64, i64, i64, vp, vp, vp, dbl, ctypes.c_int,
                                     dbl, ctypes.c_int, i64, i64,
                                     ctypes.c_int, vp, vp, vp, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_splitk_combine.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
    lib.oracle_splitk_combine.restype = ctypes.c_int
    lib.oracle_attention_bwd.argtypes = [i64, i64, i64, i64, i64, i64, vp, vp, vp, vp, dbl, ctypes.c_int,
                                         dbl, ctypes.c_int, i64, i64,
                                         ctypes.c_int, vp, vp, vp, vp, vp, vp, ctypes.c_int]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_l2norm.argtypes = [i64, i64, vp, i64, vp, vp]
    lib.oracle_l2norm.restype = ctypes.c_int
    return lib


def _f32(x) -> np.ndarray:
    """Contiguous float32 numpy copy of a numpy array or a (CPU/GPU) torch tensor."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _bias_args(bias, alibi_slopes, B, Hq, Lq, Lk):
    """(kind, bias array, element strides, slopes) for the C oracle; a dense bias
    broadcasts to [B, Hq, Lq, Lk] through zero strides."""
    kind, ba, strides, sa = BIAS_NONE, None, None, None
    if bias is not None and alibi_slopes is not None:
        raise ValueError("give either a dense bias or ALiBi slopes, not both")
    if bias is not None:
        ba = _f32(bias)
        while ba.ndim < 4:
            ba = ba[None]
        if ba.ndim != 4:
            raise ValueError("bias must have at most 4 dims")
        full = (B, Hq, Lq, Lk)
        st = []
        for dim, (n, want) in enumerate(zip(ba.shape, full)):
            if n == want:
                st.append(ba.strides[dim] // 4)
            elif n == 1:
                st.append(0)
            else:
                raise ValueError("bias shape %s does not broadcast to %s" % (ba.shape, full))
        strides = np.asarray(st, dtype=np.int64)
        kind = BIAS_DENSE
    elif alibi_slopes is not None:
        sa = _f32(alibi_slopes).reshape(-1)
        if sa.shape[0] != Hq:
            raise ValueError("need one ALiBi slope per query head")
        kind = BIAS_ALIBI
    return kind, ba, strides, sa


def attention(q, k, v, scale: float, causal: bool = False, *, bias=None,
              alibi_slopes=None, softcap: float = 0.0, window: Optional[Sequence[int]] = None,
              rows: Optional[Sequence[int]] = None, threads: Optional[int] = None, lib=None):
    """fp64 O [rows, D] and LSE [rows] of attention over q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D].

    ``bias`` is an additive score bias broadcastable to [B, Hq, Lq, Lk] (numpy or
    torch; size-1 dims broadcast).  ``alibi_slopes`` [Hq] selects the ALiBi bias
    -slope[h] * |i + Lk - Lq - j| instead.  ``softcap`` > 0 bounds the scaled
    score to softcap * tanh(score / softcap) before the bias.  ``window`` =
    (left, right) keeps only keys j with p - left <= j <= p + right, p = i + Lk
    - Lq (a negative bound is unbounded).  ``rows`` selects flat row ids
    (b*Hq + h)*Lq + i; by default every row is returned, in order, and O is
    reshaped to [B, Hq, Lq, D] and LSE to [B, Hq, Lq].
    """
    lib = lib or load()
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    B, Hq, Lq, D = qa.shape
    Bk, Hkv, Lk, Dk = ka.shape
    if va.shape != ka.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k and v")
    kind, ba, strides, sa = _bias_args(bias, alibi_slopes, B, Hq, Lq, Lk)
    ra = None
    if rows is not None:
        ra = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    n = B * Hq * Lq if ra is None else ra.shape[0]
    o = np.zeros((max(n, 0), D), dtype=np.float64)
    lse = np.zeros((max(n, 0),), dtype=np.float64)
    rc = lib.oracle_attention(B, Hq, Hkv, Lq, Lk, D, _ptr(qa), _ptr(ka), _ptr(va),
                              float(scale), int(bool(causal)), float(softcap),
                              0 if window is None else 1,
                              -1 if window is None else int(window[0]),
                              -1 if window is None else int(window[1]),
                              kind, _ptr(ba), _ptr(strides),
                              _ptr(sa), _ptr(ra), n, _ptr(o), _ptr(lse),
                              int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments (rc=%d)" % rc)
    if ra is None:
        return o.reshape(B, Hq, Lq, D), lse.reshape(B, Hq, Lq)
    return o, lse


def splitk_combine(o_part, m_part, l_part, lib=None):
    """fp64 O [..., D] and LSE [...] from partials o [..., S, D], m and l [..., S]."""
    lib = lib or load()
    oa, ma, la = _f32(o_part), _f32(m_part), _f32(l_part)
    lead = ma.shape[:-1]
    S = ma.shape[-1]
    D = oa.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    if oa.shape != tuple(lead) + (S, D) or la.shape != ma.shape:
        raise ValueError("partial shapes do not agree")
    o = np.zeros((rows, D), dtype=np.float64)
    lse = np.zeros((rows,), dtype=np.float64)
    rc = lib.oracle_splitk_combine(rows, S, D, _ptr(oa), _ptr(ma), _ptr(la), _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_splitk_combine rejected its arguments (rc=%d)" % rc)
    return o.reshape(tuple(lead) + (D,)), lse.reshape(lead)


def attention_bwd(q, k, v, dout, scale: float, causal: bool = False, *, bias=None, alibi_slopes=None,
                  softcap: float = 0.0, window: Optional[Sequence[int]] = None,
                  threads: Optional[int] = None, lib=None):
    """fp64 (dQ [B,Hq,Lq,D], dK [B,Hkv,Lk,D], dV [B,Hkv,Lk,D]) of attention for the
    output gradient ``dout``; the other arguments as for ``attention``."""
    lib = lib or load()
    qa, ka, va, da = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, Hq, Lq, D = qa.shape
    Bk, Hkv, Lk, Dk = ka.shape
    if va.shape != ka.shape or Bk != B or Dk != D or da.shape != qa.shape:
        raise ValueError("shape mismatch between q, k, v and dout")
    kind, ba, strides, sa = _bias_args(bias, alibi_slopes, B, Hq, Lq, Lk)
    dq = np.zeros((B, Hq, Lq, D), dtype=np.float64)
    dk = np.zeros((B, Hkv, Lk, D), dtype=np.float64)
    dv = np.zeros((B, Hkv, Lk, D), dtype=np.float64)
    rc = lib.oracle_attention_bwd(B, Hq, Hkv, Lq, Lk, D, _ptr(qa), _ptr(ka), _ptr(va), _ptr(da),
                                  float(scale), int(bool(causal)), float(softcap),
                                  0 if window is None else 1,
                                  -1 if window is None else int(window[0]),
                                  -1 if window is None else int(window[1]),
                                  kind, _ptr(ba), _ptr(strides), _ptr(sa),
                                  _ptr(dq), _ptr(dk), _ptr(dv), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_attention_bwd rejected its arguments (rc=%d)" % rc)
    return dq, dk, dv


def l2norm(x, lib=None):
    """fp64 (y [rows, H], norm [rows]) of the rows of the 2-D array ``x``:
    norm = sqrt(sum x^2), y = x / norm (0 for a zero row)."""
    lib = lib or load()
    xa = _f32(x)
    if xa.ndim != 2:
        raise ValueError("x must be 2-D [rows, H]")
    rows, H = xa.shape
    y = np.zeros((rows, H), dtype=np.float64)
    n = np.zeros((rows,), dtype=np.float64)
    rc = lib.oracle_l2norm(rows, H, _ptr(xa), H, _ptr(y), _ptr(n))
    if rc != 0:
        raise ValueError("oracle_l2norm rejected its arguments")
    return y, n
