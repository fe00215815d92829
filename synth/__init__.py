"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws the Q, K, V tensors and
the bias inputs that both the HIP path and the fp64 oracle consume.  Neither side
imports the other; both take their inputs from here.

Recipe (one stream per tensor):
  * Q, K, V ~ N(0, 1), drawn in fp32 by ``torch.randn`` from a ``torch.Generator``
    seeded with ``seed * 16 + tensor_id`` (Q = 0, K = 1, V = 2, dense bias = 3,
    output gradient dO = 4),
    then rounded to bf16 (round-to-nearest-even, torch's cast) when the
    workload's dtype is bf16.  The oracle receives the stored values widened
    exactly to fp32/fp64.
  * Small cases are drawn on the CPU and copied to the GPU.  Full-size cases may
    be drawn directly on the GPU with a CUDA generator (same recipe, different
    stream); the oracle then gets a host copy of exactly those stored values.
  * ALiBi slopes follow the workload definition slope_h = 2^(-8 (h + 1) / H),
    h counted from 0.

The workloads are shape stand-ins for the attention variants of the Neptune
notes (section 9: Global, Causal, ALiBi and GQA, prefill and decode, sequence
lengths 128-32768) and the Twill review's forward benchmark shape (B=4, H=32,
d=128).  No dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_BIAS, TENSOR_DOUT = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype and the score modifiers."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    dtype: str = "bf16"          # "bf16" or "f32": element type of Q, K, V
    causal: bool = False
    bias: str = "none"           # "none", "alibi" (slopes) or "dense" (tensor)
    seed: int = 0
    scale: Optional[float] = None  # None -> 1/sqrt(D) rounded to fp32
    splits: Optional[int] = None   # decode only: number of KV chunks
    softcap: float = 0.0           # > 0: cap of the scaled score
    window: Optional[tuple] = None  # (left, right) keys around each query's position
    extra: dict = field(default_factory=dict, compare=False)

    def softmax_scale(self) -> float:
        s = self.scale if self.scale is not None else self.D ** -0.5
        return float(torch.tensor(s, dtype=torch.float32).item())

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads named for this build (sizes as stated there).
C1_TINY = Workload("tiny-f32-L256-d64", 1, 1, 1, 256, 256, 64, "f32", False, "none", 1001)
C2_CAUSAL = Workload("causal-prefill-bf16-B4-H32-L4096-d128", 4, 32, 32, 4096, 4096, 128,
                     "bf16", True, "none", 1002)
C3_ALIBI = Workload("alibi-causal-prefill-bf16-B2-H16-L8192-d128", 2, 16, 16, 8192, 8192, 128,
                    "bf16", True, "alibi", 1003)
C4_DECODE = Workload("decode-splitk-gqa-bf16-B16-Hq32-Hkv8-Lk32768-d128", 16, 32, 8, 1, 32768,
                     128, "bf16", False, "none", 1004, splits=32)
C5_PREFILL = Workload("long-causal-prefill-bf16-B1-H8-L32768-d128", 1, 8, 8, 32768, 32768, 128,
                      "bf16", True, "none", 1005)
C5_DECODE = Workload("long-decode-bf16-B1-H8-Lk32768-d128", 1, 8, 8, 1, 32768, 128,
                     "bf16", False, "none", 1005)

# Config 3 with its bias given as a tensor: the same ALiBi values stored as a
# bf16 [Hq, Lq, Lk] tensor and broadcast over the batch (the dense-bias form of
# the interface), so that the bias is read from memory instead of being formed
# in registers.  Under the causal mask half of its 2 GiB is read per batch
# element.
C3_DENSE = Workload("dense-bias-causal-prefill-bf16-B2-H16-L8192-d128", 2, 16, 16, 8192, 8192, 128,
                    "bf16", True, "dense", 1003)

# The next score modifiers (SoftCap and Window of the Neptune notes, section 9),
# on shapes of the workloads above: a Gemma-style cap of 50 on the causal
# B4 H32 L4096 prefill, and a causal sliding window of 4096 keys (the query's
# own key and 4095 before it) on the long B1 H8 L32768 prefill.
SOFTCAP_PREFILL = Workload("softcap50-causal-prefill-bf16-B4-H32-L4096-d128", 4, 32, 32, 4096, 4096, 128,
                           "bf16", True, "none", 1006, softcap=50.0)
WINDOW_PREFILL = Workload("window4096-causal-prefill-bf16-B1-H8-L32768-d128", 1, 8, 8, 32768, 32768, 128,
                          "bf16", True, "none", 1007, window=(4095, -1))

# The backward pass on the shape the Twill review benchmarks it on (section
# 7.2: non-causal, batch 4, 32 heads, head dim 128; its sequence lengths run up
# to 16384), at 4096 rows, with dO ~ N(0, 1).
BWD_PREFILL = Workload("bwd-noncausal-bf16-B4-H32-L4096-d128", 4, 32, 32, 4096, 4096, 128,
                       "bf16", False, "none", 1008)

# A short-query GQA forward (16 new rows against a 32768-key cache, the group
# sizes of the Mirage lecture's GQA case, section 7.1, with 8 K/V heads): the
# shape where the choice of parallel dimensions matters most.
PLAN_SHORT_GQA = Workload("short-gqa-bf16-B1-Hq32-Hkv8-Lq16-Lk32768-d128", 1, 32, 8, 16, 32768, 128,
                          "bf16", True, "none", 1009)

# A small-grid prefill (2048 new rows of 8 heads against a 32768-key cache):
# 128 query tiles of 128 rows leave half of 256 CUs idle unless the keys are
# split as well.
PLAN_LONG_KEYS = Workload("long-keys-prefill-bf16-B1-H8-Lq2048-Lk32768-d128", 1, 8, 8, 2048, 32768, 128,
                          "bf16", True, "none", 1013)

WORKLOADS = {w.name: w for w in (C1_TINY, C2_CAUSAL, C3_ALIBI, C3_DENSE, C4_DECODE, C5_PREFILL, C5_DECODE,
                                 SOFTCAP_PREFILL, WINDOW_PREFILL, BWD_PREFILL, PLAN_SHORT_GQA, PLAN_LONG_KEYS)}


@dataclass(frozen=True)
class RowsWorkload:
    """Rows of a matrix for the row L2 norm: x ~ N(0, 1) scaled per row."""
    name: str
    rows: int
    H: int
    dtype: str
    seed: int


# The row L2 norm (the Neptune notes, sections 4 and 9, list the numerically
# stable L2 norm among the reductions of the same repair algebra): a batch of
# 32768 rows of 4096 bf16 values (one pass, rows in registers), and 8 rows of
# 4194304 fp32 values (split over the row).  Rows are N(0, 1) times 2^k with k
# cycling over -60 .. 60 in steps of 20, so magnitudes span far beyond what a
# plain fp32 sum of squares holds.
L2N_ROWS = RowsWorkload("l2norm-bf16-rows32768-H4096", 32768, 4096, "bf16", 1010)
L2N_LONG = RowsWorkload("l2norm-f32-rows8-H4194304", 8, 4194304, "f32", 1011)
ROW_WORKLOADS = {w.name: w for w in (L2N_ROWS, L2N_LONG)}


def make_rows(w: RowsWorkload, device="cpu") -> torch.Tensor:
    """x [rows, H] in the workload's dtype: N(0, 1) times 2^(20 * (r % 7) - 60) for row r."""
    x = torch.randn((w.rows, w.H), generator=_gen(w.seed, TENSOR_Q, device), device=device, dtype=torch.float32)
    k = (torch.arange(w.rows, device=device) % 7) * 20 - 60
    x *= torch.pow(2.0, k.to(torch.float32))[:, None]
    return x.to(torch_dtype(w.dtype))


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _gen(seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 16 + int(tensor_id))
    return g


def normal(shape, seed: int, tensor_id: int, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    """N(0,1) tensor of ``shape`` in the stored dtype (fp32 draw, then RNE cast)."""
    x = torch.randn(tuple(shape), generator=_gen(seed, tensor_id, device), device=device,
                    dtype=torch.float32)
    return x.to(torch_dtype(dtype))


def alibi_slopes(H: int) -> torch.Tensor:
    """slope_h = 2^(-8 (h+1) / H) for h = 0..H-1, as fp32 (CPU)."""
    h = torch.arange(H, dtype=torch.float64)
    return torch.pow(2.0, -8.0 * (h + 1.0) / H).to(torch.float32)


def alibi_bias_tensor(w: Workload, dtype: str = "bf16", device="cpu") -> torch.Tensor:
    """The ALiBi bias of the workload written out as a tensor [Hq, Lq, Lk]:
    -slope_h * |(i + Lk - Lq) - j| (query positions aligned to the end of the
    keys), formed in fp32 from the fp32 slopes and stored in ``dtype``.  An
    input, like the slopes: both the kernels and the oracle read the stored
    values."""
    sl = alibi_slopes(w.Hq).to(device)
    qpos = torch.arange(w.Lq, device=device, dtype=torch.float32) + float(w.Lk - w.Lq)
    kpos = torch.arange(w.Lk, device=device, dtype=torch.float32)
    dist = (qpos[:, None] - kpos[None, :]).abs_()
    out = torch.empty((w.Hq, w.Lq, w.Lk), dtype=torch_dtype(dtype), device=device)
    for h in range(w.Hq):
        out[h] = (dist * -sl[h]).to(out.dtype)
    return out


def make_qkv(w: Workload, device="cpu"):
    """Q [B,Hq,Lq,D], K and V [B,Hkv,Lk,D] in the workload's dtype on ``device``."""
    q = normal((w.B, w.Hq, w.Lq, w.D), w.seed, TENSOR_Q, w.dtype, device)
    k = normal((w.B, w.Hkv, w.Lk, w.D), w.seed, TENSOR_K, w.dtype, device)
    v = normal((w.B, w.Hkv, w.Lk, w.D), w.seed, TENSOR_V, w.dtype, device)
    return q, k, v


def make_dense_bias(w: Workload, shape=None, dtype: str = "f32", device="cpu") -> torch.Tensor:
    """A random additive bias, N(0,1), default shape [Hq, Lq, Lk] (broadcast over B)."""
    shape = shape if shape is not None else (w.Hq, w.Lq, w.Lk)
    return normal(shape, w.seed, TENSOR_BIAS, dtype, device)


def make_dout(w: Workload, device="cpu") -> torch.Tensor:
    """Output gradient dO [B,Hq,Lq,D], N(0,1), in the workload's dtype."""
    return normal((w.B, w.Hq, w.Lq, w.D), w.seed, TENSOR_DOUT, w.dtype, device)
