"""HIP path vs the fp64 oracle, element by element, on seeded inputs (GPU).

Sizes span several query and key tiles with ragged tails.  Tolerances:
  fp32 inputs: max |err| <= 1e-5 on O and LSE;
  bf16 inputs (fp32 accumulation): max |err| <= 1.5e-2 on O, <= 1e-3 on LSE.
Every call goes through the C ABI (the ctypes binding marshals arguments only).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import online_softmax_fusion_amd as attn

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (1.5e-2, 1e-3)}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


def compare(o_gpu, lse_gpu, O_ref, L_ref, dtype, what="", lse_tol=None, store_ulp=False):
    """The bars of the bf16 (1.5e-2 on O, 1e-3 on LSE) and fp32 inputs; with
    store_ulp, a bf16-stored O may also differ by the rounding of that store,
    half an ulp of the value (2^-8 |O|), where the same call with an fp32 O is
    held to the plain bar."""
    o_tol, l_tol = TOL[dtype]
    if lse_tol is not None:
        l_tol = lse_tol
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), what + ": non-finite O"
    err_o = float(np.max(np.abs(o - O_ref))) if o.size else 0.0
    if store_ulp and o_gpu.dtype == torch.bfloat16:
        excess = np.abs(o - O_ref) - (o_tol + 2.0 ** -8 * np.abs(O_ref))
        assert o.size == 0 or float(np.max(excess)) <= 0.0, "%s: O max abs err %.3e (bf16 store)" % (what, err_o)
    else:
        assert err_o <= o_tol, "%s: O max abs err %.3e > %.1e" % (what, err_o, o_tol)
    if lse_gpu is not None:
        l = lse_gpu.cpu().numpy().astype(np.float64)
        fin = np.isfinite(L_ref)
        assert np.array_equal(np.isfinite(l), fin), what + ": LSE infinity pattern differs"
        assert np.all(l[~fin] == -np.inf), what + ": masked rows must have LSE = -inf"
        err_l = float(np.max(np.abs(l[fin] - L_ref[fin]))) if fin.any() else 0.0
        assert err_l <= l_tol, "%s: LSE max abs err %.3e > %.1e" % (what, err_l, l_tol)
    return err_o


def inputs(B, Hq, Hkv, Lq, Lk, D, dtype, causal=False, bias="none", seed=1, qk_scale=1.0):
    w = synth.Workload("case", B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, seed)
    q, k, v = synth.make_qkv(w)
    if qk_scale != 1.0:
        q = (q.float() * qk_scale).to(q.dtype)
        k = (k.float() * qk_scale).to(k.dtype)
    gkw, okw = {}, {}
    if bias == "alibi":
        sl = synth.alibi_slopes(Hq)
        gkw["alibi_slopes"], okw["alibi_slopes"] = sl.cuda(), sl
    elif bias in ("dense_f32", "dense_bf16"):
        bt = synth.make_dense_bias(w, (Hq, Lq, Lk), "f32" if bias == "dense_f32" else "bf16")
        gkw["bias"], okw["bias"] = bt.cuda(), bt.float()
    return w, q, k, v, gkw, okw


PREFILL_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias
    (1, 1, 1, 256, 256, 64, "f32", False, "none"),        # tiny reference workload
    (2, 3, 1, 150, 333, 128, "f32", True, "none"),
    (1, 2, 2, 97, 200, 64, "f32", False, "alibi"),
    (2, 4, 4, 300, 300, 128, "bf16", True, "none"),
    (1, 4, 4, 200, 333, 128, "bf16", False, "none"),
    (2, 4, 4, 260, 260, 64, "bf16", True, "none"),
    (1, 8, 2, 190, 190, 128, "bf16", True, "none"),      # GQA
    (1, 2, 2, 100, 450, 128, "bf16", True, "none"),      # Lq < Lk, end-aligned mask
    (1, 2, 2, 300, 150, 128, "bf16", True, "none"),      # Lq > Lk: fully masked rows
    (1, 4, 4, 257, 257, 128, "bf16", True, "alibi"),
    (2, 2, 2, 130, 190, 128, "bf16", False, "alibi"),
    (2, 2, 2, 96, 140, 128, "bf16", False, "dense_f32"),
    (1, 2, 2, 129, 129, 64, "bf16", True, "dense_bf16"),
    # >= 1024 rows that see >= 4096 keys on average, on a grid too small for
    # the eight-wave form (the four-wave kernel over long rows)
    (1, 2, 1, 1100, 4200, 128, "bf16", False, "none"),
    (1, 2, 2, 1030, 4500, 128, "bf16", False, "alibi"),
    (1, 1, 1, 1300, 6000, 128, "bf16", True, "dense_f32"),
    (1, 1, 1, 1, 77, 128, "bf16", False, "none"),
    (1, 2, 1, 33, 1, 128, "bf16", True, "none"),
    # causal work order: with 2 query tiles per head, 32 heads fill each XCD's
    # range with windows of 4 heads, 16 heads with windows of 2 (8 waves: 5
    # query tiles per head, windows of 2)
    (2, 16, 4, 250, 250, 128, "bf16", True, "none"),
    (1, 16, 16, 200, 230, 128, "bf16", True, "alibi"),
    (1, 16, 4, 1030, 5150, 128, "bf16", True, "none"),
    # causal ALiBi (the bias folded into the scores by one more matrix product):
    # d = 64, end-aligned Lq < Lk, Lq > Lk (rows that see no key), GQA
    (2, 4, 4, 260, 260, 64, "bf16", True, "alibi"),
    (1, 4, 2, 150, 700, 128, "bf16", True, "alibi"),
    (1, 2, 2, 300, 140, 128, "bf16", True, "alibi"),
]


# The eight-wave (256-row) workgroup: >= 1024 rows that see >= 4096 keys on
# average (>= 8192 when causal), with at least one 256-row workgroup per CU
# (B * Hq * ceil(Lq / 256) = 320 here).  Compared on sampled rows: the tile
# edges of every 256-row block, the ragged last block, in every head.  The
# causal cases run windows of 4 heads (8 heads per XCD).
EIGHT_WAVE_CASES = [
    # B, Hq, Hkv, Lq, Lk, causal, bias
    (1, 64, 16, 1030, 4200, False, "none"),
    (1, 64, 64, 1030, 4500, False, "alibi"),
    (1, 64, 16, 1030, 8800, True, "dense_f32"),
    (1, 64, 8, 1030, 8900, True, "none"),
    (1, 64, 16, 1030, 8800, True, "dense_bf16"),   # bf16 bias tiles through LDS
]


@pytest.mark.parametrize("case", EIGHT_WAVE_CASES, ids=[str(i) for i in range(len(EIGHT_WAVE_CASES))])
def test_prefill_eight_wave_sampled(case):
    B, Hq, Hkv, Lq, Lk, causal, bias = case
    print("eight-wave prefill case", case, flush=True)
    w = synth.Workload("case8", B, Hq, Hkv, Lq, Lk, 128, "bf16", causal, bias, 29)
    q, k, v = synth.make_qkv(w)
    gkw, okw = {}, {}
    if bias == "alibi":
        sl = synth.alibi_slopes(Hq)
        gkw["alibi_slopes"], okw["alibi_slopes"] = sl.cuda(), sl
    elif bias in ("dense_f32", "dense_bf16"):
        bt = synth.make_dense_bias(w, (Lq, Lk), bias[6:])   # broadcast over batch and heads
        gkw["bias"], okw["bias"] = bt.cuda(), bt.float()
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), causal, **gkw)
    torch.cuda.synchronize()
    local = sorted({i for t in range(0, Lq, 256) for i in (t, t + 1, t + 127, t + 128, t + 255) if i < Lq} | {Lq - 1})
    rows = np.array([(b * Hq + h) * Lq + i for b in range(B) for h in range(Hq) for i in local], dtype=np.int64)
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, rows=rows, **okw)
    compare(o.reshape(-1, 128)[torch.from_numpy(rows).cuda()], lse.reshape(-1)[torch.from_numpy(rows).cuda()],
            O_ref, L_ref, "bf16", str(case))


# bf16 dense bias at d = 128: rows of contiguous keys that start 16-byte
# aligned are loaded a tile at a time into LDS beside K and V (eight-wave
# workgroups); other layouts read each element where it is used.  Layouts:
# contiguous [Hq, Lq, Lk] (shared by the batch); rows padded to a longer stride
# (the keys past Lk in a row's last chunk are padding); one [Lq, Lk] plane
# broadcast over batch and heads; a plane per batch element; rows whose stride
# is not a multiple of 8 elements (the per-element path).
DENSE_BF16_CASES = [
    # B, Hq, Hkv, Lq, Lk, causal, layout
    (2, 4, 2, 300, 328, True, "contiguous"),
    (1, 3, 3, 520, 330, False, "padded"),
    (2, 2, 1, 700, 512, True, "broadcast"),
    (1, 2, 2, 600, 200, True, "contiguous"),    # Lq > Lk: rows that see no key
    (1, 2, 2, 100, 333, False, "contiguous"),   # stride of 333 elements: per-element path
    (1, 2, 2, 1, 64, False, "contiguous"),
    (3, 2, 2, 260, 264, False, "contiguous"),   # three batch elements share the bias (work order)
    (2, 2, 2, 260, 264, True, "batched"),       # [B, Hq, Lq, Lk]: a bias plane per batch element
]


@pytest.mark.parametrize("case", DENSE_BF16_CASES, ids=[str(i) for i in range(len(DENSE_BF16_CASES))])
def test_prefill_dense_bf16_layouts(case):
    B, Hq, Hkv, Lq, Lk, causal, layout = case
    print("dense bf16 bias case", case, flush=True)
    w = synth.Workload("dense", B, Hq, Hkv, Lq, Lk, 128, "bf16", causal, "dense", 31 + Lq)
    q, k, v = synth.make_qkv(w)
    if layout == "broadcast":
        bt = synth.make_dense_bias(w, (Lq, Lk), "bf16")
    elif layout == "batched":
        bt = synth.make_dense_bias(w, (B, Hq, Lq, Lk), "bf16")
    elif layout == "padded":
        bt = synth.make_dense_bias(w, (Hq, Lq, Lk + 6), "bf16")[..., :Lk]
    else:
        bt = synth.make_dense_bias(w, (Hq, Lq, Lk), "bf16")
    bg = bt.cuda() if layout != "padded" else synth.make_dense_bias(w, (Hq, Lq, Lk + 6), "bf16").cuda()[..., :Lk]
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), causal, bias=bg)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, bias=bt.float())
    compare(o, lse, O_ref, L_ref, "bf16", str(case))


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(i) for i in range(len(PREFILL_CASES))])
def test_prefill_parity(case):
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias = case
    w, q, k, v, gkw, okw = inputs(B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, seed=17 + len(str(case)))
    print("prefill case", case, flush=True)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), causal, **gkw)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, **okw)
    compare(o, lse, O_ref, L_ref, dtype, str(case))


# SoftCap and sliding Window (the readings of the oracle: cap on the scaled
# score before the bias; keys p - left <= j <= p + right, negative = unbounded)
MOD_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, softcap, window
    (1, 4, 4, 300, 300, 128, "bf16", True, "none", 0.0, (64, -1)),     # causal sliding window
    (1, 2, 2, 200, 333, 128, "bf16", True, "none", 0.0, (100, 0)),     # Lq < Lk
    (2, 2, 1, 257, 257, 128, "bf16", False, "none", 0.0, (70, 30)),    # two-sided, unaligned
    (1, 2, 2, 260, 260, 64, "bf16", True, "none", 0.0, (0, 0)),        # only the diagonal
    (1, 2, 2, 300, 150, 128, "bf16", True, "none", 0.0, (40, -1)),     # Lq > Lk: empty rows
    (1, 2, 2, 190, 190, 128, "bf16", False, "none", 0.0, (-1, 5)),     # right bound only
    (1, 4, 4, 256, 256, 128, "bf16", True, "none", 2.0, None),         # soft cap
    (2, 2, 2, 130, 190, 128, "bf16", False, "alibi", 5.0, None),       # cap + ALiBi
    (1, 2, 2, 129, 129, 64, "bf16", True, "dense_bf16", 3.0, (20, -1)),  # cap + bias + window
    (1, 2, 2, 160, 160, 128, "bf16", True, "none", 30.0, (50, -1)),    # loose cap + window
    (1, 2, 2, 150, 333, 128, "f32", True, "none", 4.0, (60, -1)),      # fp32 path
    (1, 2, 2, 97, 200, 64, "f32", False, "alibi", 1.5, (10, 10)),
    (1, 4, 4, 300, 420, 128, "bf16", True, "alibi", 0.0, (90, -1)),    # causal ALiBi + window (folded form)
    (1, 4, 4, 300, 320, 128, "bf16", True, "dense_bf16", 0.0, (90, -1)),  # bias tiles, keys descending
    (2, 4, 4, 300, 320, 128, "bf16", True, "dense_bf16", 0.0, (90, -1)),  # the same, bias shared by two batch elements
    (1, 2, 2, 260, 264, 128, "bf16", False, "dense_bf16", 0.0, (70, 30)),  # bias tiles, keys ascending
    (1, 4, 4, 300, 300, 128, "bf16", True, "none", 64.0, None),        # largest cap of the exp-only form
    (1, 4, 4, 300, 300, 128, "bf16", True, "none", 64.5, None),        # smallest cap of the exact form
]


@pytest.mark.parametrize("case", MOD_CASES, ids=[str(i) for i in range(len(MOD_CASES))])
def test_prefill_softcap_window_parity(case):
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, softcap, window = case
    w, q, k, v, gkw, okw = inputs(B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, seed=61 + Lq, qk_scale=2.0)
    print("prefill softcap/window case", case, flush=True)
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, softcap=softcap, window=window, **okw)
    # the scores are scaled up here (peaky rows, |O| up to about 3): the
    # arithmetic is held to the bar on an fp32 O, the default bf16 O to the bar
    # plus the rounding of its store
    for od in ((torch.float32, None) if dtype == "bf16" else (None,)):
        o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), causal, softcap=softcap,
                                       window=window, out_dtype=od, **gkw)
        torch.cuda.synchronize()
        compare(o, lse, O_ref, L_ref, dtype, "%s out %s" % (case, od), store_ulp=True)


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, softcap, window, splits
    (2, 8, 2, 1, 1000, 128, "bf16", False, "none", 0.0, (300, -1), 4),   # chunks outside the window
    (1, 4, 4, 1, 777, 128, "bf16", True, "none", 3.0, (100, 0), 3),
    (1, 16, 2, 5, 700, 128, "bf16", True, "alibi", 5.0, (64, -1), 6),  # 40 stacked rows
    (2, 4, 2, 1, 300, 64, "bf16", False, "dense_f32", 2.0, None, 3),
    (1, 4, 2, 1, 500, 128, "f32", False, "none", 4.0, (50, -1), 4),
    (1, 2, 2, 3, 300, 64, "f32", True, "alibi", 0.0, (0, 0), 2),
], ids=[str(i) for i in range(6)])
def test_decode_softcap_window_parity(case):
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, softcap, window, S = case
    w, q, k, v, gkw, okw = inputs(B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, seed=91 + S, qk_scale=2.0)
    print("decode softcap/window case", case, flush=True)
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), S, w.softmax_scale(), causal, softcap=softcap,
                         window=window, out_dtype=torch.float32, **gkw)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, softcap=softcap, window=window, **okw)
    compare(o, lse, O_ref, L_ref, dtype, str(case))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("cap", [10.0, 50.0])
def test_prefill_softcap_polynomial_and_exact_tiles(causal, cap):
    """The prefill kernel forms the soft cap as a polynomial on key tiles whose
    raw scores all lie within |scale s| <= cap / 2 and by the exp form on the
    others; keys 128..191 and 320..383 are scaled up so that both kinds of tile
    (and the growth of the running maximum between them) occur in one row."""
    w, q, k, v, gkw, okw = inputs(1, 4, 2, 450, 450, 128, "bf16", causal, "none", seed=77)
    kf = k.float()
    kf[:, :, 128:192] *= 8.0
    kf[:, :, 320:384] *= 5.0
    k = kf.to(torch.bfloat16)
    print("prefill softcap poly/exact case", causal, cap, flush=True)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), causal, softcap=cap)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, softcap=cap)
    compare(o, lse, O_ref, L_ref, "bf16", "softcap %g causal %s" % (cap, causal))


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Lq, Lk, D, causal, cap, window, scale
    (1, 8, 2, 190, 333, 64, False, 30.0, None, 0.2),      # GQA, d = 64, non-default scale
    (2, 4, 4, 260, 260, 64, True, 20.0, (70, -1), None),   # d = 64, window
    (1, 4, 1, 300, 450, 128, True, 64.0, (100, 20), 0.15),  # largest cap of the form, two-sided window
], ids=["gqa_d64", "d64_window", "d128_window"])
def test_prefill_softcap_polynomial_shapes(case):
    """The polynomial soft cap on other shapes: GQA, d = 64, a non-default
    scale (which moves the polynomial's range) and sliding windows."""
    B, Hq, Hkv, Lq, Lk, D, causal, cap, window, scale = case
    w, q, k, v, gkw, okw = inputs(B, Hq, Hkv, Lq, Lk, D, "bf16", causal, "none", seed=79 + Lq)
    sc = w.softmax_scale() if scale is None else scale
    print("prefill softcap shape case", case, flush=True)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), sc, causal, softcap=cap, window=window)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, sc, causal, softcap=cap, window=window)
    compare(o, lse, O_ref, L_ref, "bf16", str(case))


def test_prefill_tiny_softcap():
    """A cap so small against the scale (1e-8) that the polynomial's scaled
    coefficients leave the float range: every tile takes the exp form, and
    the rows average the values they see."""
    w, q, k, v, gkw, okw = inputs(1, 2, 2, 200, 200, 128, "bf16", True, "none", seed=78)
    print("prefill tiny softcap", flush=True)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), True, softcap=1e-8)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), True, softcap=1e-8)
    compare(o, lse, O_ref, L_ref, "bf16", "softcap 1e-8")


def test_unbounded_window_and_huge_cap_match_plain():
    """A window wider than the keys and a cap far above every score give the
    plain kernel's result (up to the cap's rounding)."""
    w, q, k, v, _, _ = inputs(1, 4, 4, 200, 200, 128, "bf16", True, seed=5)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    o0, l0 = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), True)
    o1, l1 = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), True, window=(1000, 1000))
    o2, l2 = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), True, softcap=1e6)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert float((o2.float() - o0.float()).abs().max()) <= 1.6e-2
    assert float((l2 - l0).abs().max()) <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_fp32_output(dtype):
    w, q, k, v, _, _ = inputs(1, 2, 2, 140, 140, 128, dtype, True)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), True,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), True)
    err = compare(o, lse, O_ref, L_ref, dtype, "fp32 out")
    if dtype == "bf16":
        assert err <= 8e-3   # no final bf16 rounding of O


def test_prefill_strided_views():
    """q/k/v as views of a packed [B, L, 3, H, D] buffer (non-contiguous b/h/l strides)."""
    B, H, L, D = 2, 4, 150, 128
    w = synth.Workload("packed", B, H, H, L, L, D, "bf16", True, "none", 5)
    packed = synth.normal((B, L, 3, H, D), 5, 0, "bf16")
    q, k, v = (packed[:, :, t].permute(0, 2, 1, 3) for t in range(3))
    g = packed.cuda()
    qg, kg, vg = (g[:, :, t].permute(0, 2, 1, 3) for t in range(3))
    o, lse = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), True)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), True)
    compare(o, lse, O_ref, L_ref, "bf16", "strided")


def test_prefill_empty_keys():
    q = synth.normal((1, 2, 40, 128), 3, 0, "bf16").cuda()
    k = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = attn.attn_fwd_prefill(q, k, k, 0.1, False)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_prefill_large_logits():
    """q and K scaled by 40 (Mirage lecture notes, section 5.5): logits in the
    thousands stay finite.  LSE is compared relative to its magnitude: the
    fp32 score of a length-128 dot product of size ~1e4 carries ~1e-3 absolute
    rounding; O and the relative LSE error keep the bf16 bars."""
    w, q, k, v, _, _ = inputs(1, 2, 2, 130, 130, 128, "bf16", True, qk_scale=40.0, seed=9)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), True)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), True)
    assert np.max(np.abs(L_ref)) > 500
    compare(o, lse, O_ref, L_ref, "bf16", "large logits",
            lse_tol=1e-5 * float(np.max(np.abs(L_ref))) + 1e-3)


def test_prefill_constant_v():
    w, q, k, _, _, _ = inputs(1, 2, 2, 200, 200, 128, "bf16", True, seed=21)
    v = torch.full(k.shape, 0.75, dtype=torch.bfloat16)
    o, _ = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), True)
    torch.cuda.synchronize()
    assert float((o.float() - 0.75).abs().max()) <= 1.5e-2


@pytest.mark.parametrize("causal,Lq,Lk", [(True, 300, 300), (True, 200, 460), (False, 260, 300)])
def test_alibi_matches_dense_bias_of_its_values(causal, Lq, Lk):
    """ALiBi from the slopes (under a causal mask the folded form, whose bias
    enters through one more matrix product) against the same values given as a
    dense fp32 bias: the two paths agree within the bf16 bars; and slopes of 0
    give the unbiased result."""
    w, q, k, v, _, _ = inputs(1, 4, 4, Lq, Lk, 128, "bf16", causal, "alibi", seed=8 + Lq)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    sl = synth.alibi_slopes(4)
    dense = synth.alibi_bias_tensor(w.with_(bias="dense"), "f32").cuda()
    o_a, l_a = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), causal, alibi_slopes=sl.cuda(),
                                     out_dtype=torch.float32)
    o_d, l_d = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), causal, bias=dense, out_dtype=torch.float32)
    o_0, l_0 = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), causal, alibi_slopes=torch.zeros(4).cuda(),
                                     out_dtype=torch.float32)
    o_n, l_n = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    fin = torch.isfinite(l_a)
    assert torch.equal(fin, torch.isfinite(l_d))
    assert float((o_a - o_d).abs().max()) <= 1.5e-2
    assert float((l_a[fin] - l_d[fin]).abs().max()) <= 1e-3
    assert float((o_0 - o_n).abs().max()) <= 1.5e-2
    assert float((l_0[fin] - l_n[fin]).abs().max()) <= 1e-3


# Slopes beyond ALiBi's own (which are at most 1), of both signs.  Under a
# causal mask the bias is folded into the key-query product relative to the
# position of each wave's first row, so the rounding it adds grows with the
# slope; up to |slope| = 64 it stays inside the bf16 bars.  Checked in the
# four-wave and eight-wave workgroups (the correction of each wave's row
# constant) and in the split form (the per-chunk reference values).
SLOPE_RANGE = [0.5, 8.0, 64.0, -0.05]


def _slopes(Hq):
    return torch.tensor([SLOPE_RANGE[h % len(SLOPE_RANGE)] for h in range(Hq)], dtype=torch.float32)


def test_folded_alibi_slope_range_four_waves():
    w, q, k, v, _, _ = inputs(1, 4, 4, 300, 330, 128, "bf16", True, "alibi", seed=61)
    sl = _slopes(4)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), True, alibi_slopes=sl.cuda())
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), True, alibi_slopes=sl)
    compare(o, lse, O_ref, L_ref, "bf16", "slopes %s" % SLOPE_RANGE)


def test_folded_alibi_slope_range_split():
    w, q, k, v, _, _ = inputs(1, 4, 4, 200, 1500, 128, "bf16", True, "alibi", seed=62)
    sl = _slopes(4)
    op, mp, lp = attn.attn_fwd_prefill_splitk(q.cuda(), k.cuda(), v.cuda(), 3, w.softmax_scale(), True,
                                              alibi_slopes=sl.cuda())
    o, lse = attn.attn_splitk_combine(op, mp, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), True, alibi_slopes=sl)
    compare(o, lse, O_ref, L_ref, "bf16", "split, slopes %s" % SLOPE_RANGE)


def test_folded_alibi_slope_range_eight_waves():
    B, Hq, Hkv, Lq, Lk = 1, 64, 8, 1030, 8900   # eight-wave workgroups (as in the sampled cases above)
    w = synth.Workload("case8", B, Hq, Hkv, Lq, Lk, 128, "bf16", True, "alibi", 63)
    q, k, v = synth.make_qkv(w)
    sl = _slopes(Hq)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), True, alibi_slopes=sl.cuda())
    torch.cuda.synchronize()
    # the first rows of all eight waves of the first and last 256-row blocks, their neighbours
    local = sorted({i for t in (0, 768, 1024) for i in range(t, min(t + 256, Lq), 31)} | {Lq - 1})
    rows = np.array([h * Lq + i for h in range(Hq) for i in local], dtype=np.int64)
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), True, rows=rows, alibi_slopes=sl)
    idx = torch.from_numpy(rows).cuda()
    compare(o.reshape(-1, 128)[idx], lse.reshape(-1)[idx], O_ref, L_ref, "bf16", "eight waves, slopes")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("growth", [0.15, -0.15, 0.01])
def test_prefill_running_max_growth(causal, growth):
    """Scores that move steadily along the keys: s_ij ~ growth * j (natural
    units) for every row.  Rising by ~9.6 per 64-key tile, the running maximum
    outgrows the lazy threshold on every tile (the weights are re-formed after
    a repair); falling, only the first tile sets it; rising slowly, the weights
    of a tile sum past 2^8 without any single one passing it."""
    B, H, Lq, Lk, D = 1, 2, 130, 520, 128
    g = torch.Generator().manual_seed(71)
    q0 = torch.randn(H, 1, D, generator=g)
    q = (q0 + 0.01 * torch.randn(H, Lq, D, generator=g)).unsqueeze(0)
    scale = 1.0 / math.sqrt(D)
    unit = q0 / (q0.pow(2).sum(-1, keepdim=True) * scale)        # <q0, unit> * scale = 1
    j = torch.arange(Lk, dtype=torch.float32).view(1, Lk, 1)
    k = (growth * j * unit + 0.05 * torch.randn(H, Lk, D, generator=g)).unsqueeze(0)
    v = torch.randn(B, H, Lk, D, generator=g)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), scale, causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, scale, causal)
    compare(o, lse, O_ref, L_ref, "bf16", "growth %g causal %s" % (growth, causal))


def test_prefill_deterministic():
    w, q, k, v, _, _ = inputs(1, 4, 4, 300, 300, 128, "bf16", True, "alibi", seed=4)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    sl = synth.alibi_slopes(4).cuda()
    a = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), True, alibi_slopes=sl)
    b = attn.attn_fwd_prefill(qg, kg, vg, w.softmax_scale(), True, alibi_slopes=sl)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------------------
# split-K decode
# ----------------------------------------------------------------------------
DECODE_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, splits
    (2, 8, 2, 1, 1000, 128, "bf16", False, "none", 3),
    (2, 8, 2, 1, 1000, 128, "bf16", False, "none", 32),
    (1, 4, 4, 1, 777, 128, "bf16", False, "none", 1),
    (1, 4, 4, 1, 100, 128, "bf16", False, "none", 10),     # empty trailing chunks
    (3, 32, 8, 1, 2048, 128, "bf16", False, "none", 4),
    (1, 16, 2, 5, 700, 128, "bf16", True, "none", 6),       # 40 stacked rows: two row blocks
    (1, 4, 1, 1, 999, 64, "bf16", False, "alibi", 5),
    (2, 4, 2, 1, 300, 128, "bf16", False, "dense_f32", 3),
    (1, 4, 2, 1, 500, 128, "f32", False, "none", 4),
    (1, 2, 2, 3, 300, 64, "f32", True, "alibi", 2),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(i) for i in range(len(DECODE_CASES))])
def test_decode_parity(case):
    B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, S = case
    w, q, k, v, gkw, okw = inputs(B, Hq, Hkv, Lq, Lk, D, dtype, causal, bias, seed=31 + S)
    print("decode case", case, flush=True)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    op, mp, lp = attn.attn_fwd_decode_splitk(qg, kg, vg, S, w.softmax_scale(), causal, **gkw)
    o, lse = attn.attn_splitk_combine(op, mp, lp, out_dtype=q.dtype)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, **okw)
    compare(o, lse, O_ref, L_ref, dtype, "decode " + str(case))

    # the combine kernel against the fp64 combine of the same partials
    Oc, Lc = oracle.splitk_combine(op.cpu(), mp.cpu(), lp.cpu())
    compare(attn.attn_splitk_combine(op, mp, lp, out_dtype=torch.float32)[0], lse, Oc, Lc, "f32",
            "combine vs fp64 combine")

    # each chunk's partial against the oracle restricted to that chunk
    C = attn.chunk_length(Lk, S)
    opc, mpc, lpc = op.cpu().double().numpy(), mp.cpu().double().numpy(), lp.cpu().double().numpy()
    bias_t = okw.get("bias")
    for s in range(S):
        lo, hi = s * C, min((s + 1) * C, Lk)
        if hi <= lo:
            assert np.all(np.isneginf(mpc[..., s])) and np.all(lpc[..., s] == 0) and np.all(opc[..., s, :] == 0)
            continue
        # the chunk seen as its own attention problem: keep each row's position
        # by shifting it with a dense mask equal to the original visibility
        pos = np.arange(Lq)[:, None] + (Lk - Lq)
        keys = np.arange(lo, hi)[None, :]
        extra = np.zeros((Hq, Lq, hi - lo))
        if causal:
            extra = np.where(keys > pos, -np.inf, 0.0)[None].repeat(Hq, 0)
        if "alibi_slopes" in okw:
            sl = okw["alibi_slopes"].double().numpy()
            extra = extra - sl[:, None, None] * np.abs(pos - keys)[None]
        if bias_t is not None:
            extra = extra + bias_t.double().numpy()[:, :, lo:hi]
        Os, Ls = oracle.attention(q, k[:, :, lo:hi], v[:, :, lo:hi], w.softmax_scale(), False,
                                  bias=extra.astype(np.float32))
        l_s, m_s = lpc[..., s], mpc[..., s]
        fin = np.isfinite(Ls)
        assert np.array_equal(np.isfinite(m_s), fin)
        got_lse = m_s[fin] + np.log(l_s[fin])
        assert np.max(np.abs(got_lse - Ls[fin])) <= TOL[dtype][1], "chunk %d LSE" % s
        got_o = opc[..., s, :][fin] / l_s[fin][:, None]
        assert np.max(np.abs(got_o - Os[fin])) <= (1e-5 if dtype == "f32" else 1e-2), "chunk %d O" % s


def test_decode_gqa_equals_repeated_heads():
    w, q, k, v, _, _ = inputs(2, 8, 2, 1, 1500, 128, "bf16", seed=12)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    a = attn.decode(qg, kg, vg, 4, w.softmax_scale())
    b = attn.decode(qg, kg.repeat_interleave(4, 1).contiguous(), vg.repeat_interleave(4, 1).contiguous(), 4,
                    w.softmax_scale())
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("S", [1, 2, 4, 32])
def test_decode_split_count_invariance(S):
    """Split-K over any number of chunks equals the unsplit result (Neptune
    notes section 6; Mirage lecture notes section 5.5, four chunks)."""
    w, q, k, v, _, _ = inputs(1, 4, 4, 1, 1024, 128, "bf16", seed=40)
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), S, w.softmax_scale(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale())
    compare(o, lse, O_ref, L_ref, "bf16", "S=%d" % S)


def test_decode_deterministic():
    w, q, k, v, _, _ = inputs(2, 8, 2, 1, 3000, 128, "bf16", seed=8)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    a = attn.decode(qg, kg, vg, 7, w.softmax_scale())
    b = attn.decode(qg, kg, vg, 7, w.softmax_scale())
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_choose_splits_on_device():
    cu = attn.attn_device_cu_count(0)
    assert cu > 0
    S = attn.attn_decode_choose_splits(1, 8, 8, 1, 32768, cu)
    w, q, k, v, _, _ = inputs(1, 8, 8, 1, 4096, 128, "bf16", seed=2)
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), None, w.softmax_scale())
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale())
    compare(o, lse, O_ref, L_ref, "bf16", "auto splits")
    assert S >= 1


@pytest.mark.parametrize("rows_shape,D,S", [((8, 64, 5), 128, 3), ((3, 40, 20), 64, 33), ((1, 2, 1), 128, 70)])
def test_combine_parity_synthetic_partials(rows_shape, D, S):
    """The combine alone on synthetic partials (both launch shapes: few rows
    and > 2048 rows), with empty chunks (m = -inf) and whole rows without keys,
    against the fp64 combine of the oracle."""
    B, Hq, Lq = rows_shape
    print("combine case", rows_shape, D, S, flush=True)
    g = torch.Generator().manual_seed(B * 1000 + Hq * 10 + S)
    op = torch.randn((B, Hq, Lq, S, D), generator=g)
    mp = 3.0 * torch.randn((B, Hq, Lq, S), generator=g)
    lp = torch.rand((B, Hq, Lq, S), generator=g) * 50 + 0.5
    empty = torch.rand((B, Hq, Lq, S), generator=g) < 0.2
    mp[empty] = -math.inf
    lp[empty] = 0.0
    op[empty] = 0.0
    mp[0, 0, 0, :] = -math.inf           # a row that saw no key at all
    lp[0, 0, 0, :] = 0.0
    op[0, 0, 0, :, :] = 0.0
    o, lse = attn.attn_splitk_combine(op.cuda(), mp.cuda(), lp.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    Oc, Lc = oracle.splitk_combine(op, mp, lp)
    compare(o, lse, Oc, Lc, "f32", "combine %s" % (rows_shape,))
    assert torch.all(o[0, 0, 0] == 0) and lse[0, 0, 0].item() == -math.inf


def test_decode_graph_replay():
    """The decode step (local step + combine) captured in a HIP graph gives the
    eager result on every replay, with other eager work between replays."""
    w, q, k, v, _, _ = inputs(2, 8, 2, 1, 3000, 128, "bf16", seed=9)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    S = 6
    op = torch.empty((2, 8, 1, S, 128), dtype=torch.float32, device="cuda")
    mp = torch.empty((2, 8, 1, S), dtype=torch.float32, device="cuda")
    lp = torch.empty_like(mp)
    o = torch.empty_like(qg)
    lse = torch.empty((2, 8, 1), dtype=torch.float32, device="cuda")

    def step():
        attn.attn_fwd_decode_splitk(qg, kg, vg, S, w.softmax_scale(), o_part=op, m_part=mp, l_part=lp)
        attn.attn_splitk_combine(op, mp, lp, out=o, lse=lse)

    step()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        o.zero_()
        lse.zero_()
        attn.decode(qg * 0.5, kg, vg, 3, w.softmax_scale())   # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "replay %d" % r
