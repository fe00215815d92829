"""Backward pass (attn_bwd) vs the fp64 oracle's gradients, on seeded inputs (GPU).

The HIP backward consumes the HIP forward's O and LSE, as a caller would; the
oracle recomputes everything from Q, K, V and dO in fp64.  Sizes span several
64-row tiles and 128-key workgroups with ragged tails.

Tolerance (bf16 inputs, fp32 accumulation).  The kernels round two kinds of
values to bf16 (unit roundoff u = 2^-8) before a product: the weights P (for
dV) and dS (for dK and dQ); Delta = <dO, O> also carries the bf16 rounding of
the stored O.  Each gradient element is a sum of n such rounded terms, so its
error is at most u * sum |terms| and, with independent rounding signs, about
u * sqrt(sum terms^2): a relative Frobenius error of order u/2.  Measured on
these cases: max |err| <= 6e-3 * max |ref| (bf16 outputs, which add up to u/2
relative per element; 4.7e-3 with fp32 outputs) and a relative Frobenius
error <= 2.6e-3.  The test allows max |err| <= 2e-2 * max |ref| per tensor
(about 5 u) and a relative Frobenius error <= 8e-3 (2 u).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import online_softmax_fusion_amd as attn

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
FRO_REL = 8e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


def grad_errors(got, ref):
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), "non-finite gradient"
    if ref.size == 0:
        return 0.0, 0.0
    scale = float(np.max(np.abs(ref)))
    err = np.abs(g - ref)
    if scale == 0.0:
        return float(np.max(err)), float(np.max(err))
    return float(np.max(err)) / scale, float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))


def check_grads(got, refs, what):
    out = []
    # a key no query row sees (dV_j = sum_i P_ij dO_i is exactly 0 in the
    # oracle only then) must get exactly 0 in dK and dV
    dead = np.all(refs[2] == 0.0, axis=-1)
    if dead.any():
        for name, g in (("dk", got[1]), ("dv", got[2])):
            gd = g.float().cpu().numpy()[dead]
            assert np.all(gd == 0.0), "%s %s: %d keys no row sees are not zero" % (what, name, int(dead.sum()))
    for name, g, r in zip(("dq", "dk", "dv"), got, refs):
        mx, fro = grad_errors(g, r)
        print("%s %s: max|err|/max|ref| %.2e  fro %.2e" % (what, name, mx, fro), flush=True)
        assert mx <= MAX_REL, "%s %s: max err %.3e of max|ref| > %.1e" % (what, name, mx, MAX_REL)
        assert fro <= FRO_REL, "%s %s: relative Frobenius err %.3e > %.1e" % (what, name, fro, FRO_REL)
        out.append((mx, fro))
    return out


def make_case(B, Hq, Hkv, Lq, Lk, D, causal=False, bias="none", softcap=0.0, window=None, seed=7,
              scale=None):
    w = synth.Workload("bwd-case", B, Hq, Hkv, Lq, Lk, D, "bf16", causal, bias, seed, scale=scale,
                       softcap=softcap, window=window)
    q, k, v = synth.make_qkv(w)
    do = synth.make_dout(w)
    gkw, okw = {}, {}
    if bias == "alibi":
        sl = synth.alibi_slopes(Hq)
        gkw["alibi_slopes"], okw["alibi_slopes"] = sl.cuda(), sl
    elif bias in ("dense_f32", "dense_bf16", "dense_inf"):
        bt = synth.make_dense_bias(w, (Hq, Lq, Lk), "bf16" if bias == "dense_bf16" else "f32")
        if bias == "dense_inf":
            bt[:, 0, :] = -math.inf                   # a row with no usable key
            bt[:, 3, ::3] = -math.inf
        gkw["bias"], okw["bias"] = bt.cuda(), bt.float()
    return w, q, k, v, do, gkw, okw


def run_case(w, q, k, v, do, gkw, okw, grad_dtype=torch.float32):
    scale = w.softmax_scale()
    qg, kg, vg, dg = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.attn_fwd_prefill(qg, kg, vg, scale, w.causal, softcap=w.softcap, window=w.window, **gkw)
    got = attn.attn_bwd(qg, kg, vg, o, lse, dg, scale, w.causal, softcap=w.softcap, window=w.window,
                        grad_dtype=grad_dtype, **gkw)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(q.float(), k.float(), v.float(), do.float(), scale, w.causal,
                                softcap=w.softcap, window=w.window, **okw)
    return got, refs


BWD_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, bias, softcap, window
    (1, 2, 2, 200, 200, 128, True, "none", 0.0, None),
    (2, 4, 2, 130, 257, 64, False, "none", 0.0, None),          # GQA, Lq != Lk, D = 64
    (1, 4, 1, 96, 160, 128, True, "none", 0.0, None),           # G = 4, causal with Lq < Lk
    (1, 2, 2, 150, 150, 128, True, "alibi", 0.0, None),
    (1, 4, 2, 170, 290, 128, False, "alibi", 0.0, None),       # paired dK/dV with ALiBi, keys on both sides
    (1, 2, 2, 160, 200, 128, True, "alibi", 6.0, (50, -1)),    # ALiBi + cap + window, paired dK/dV
    (1, 2, 1, 100, 140, 64, False, "dense_inf", 0.0, None),     # -inf bias entries, a dead row
    (2, 2, 2, 96, 190, 128, False, "dense_bf16", 0.0, None),
    (1, 2, 2, 180, 180, 128, True, "none", 5.0, None),          # soft cap
    (1, 2, 2, 230, 230, 128, True, "none", 0.0, (40, 0)),       # causal sliding window
    (1, 2, 1, 120, 300, 64, False, "alibi", 0.0, (20, 15)),     # two-sided window, GQA
    (1, 2, 2, 200, 200, 128, False, "dense_f32", 8.0, (64, 64)),  # cap + window + dense bias
    (1, 2, 2, 300, 150, 128, True, "none", 0.0, None),          # Lq > Lk: rows without keys
    (1, 1, 1, 1, 77, 128, False, "none", 0.0, None),            # one query row
    (1, 2, 1, 33, 1, 128, True, "none", 0.0, None),             # one key
    # keys below Lk - Lq - left are seen by no row; the 32-key block of keys
    # 128-159 holds such keys and seen ones (their dK, dV must be exactly 0)
    (1, 2, 2, 142, 305, 128, True, "none", 0.0, (7, 9)),
    (1, 4, 2, 100, 300, 64, False, "dense_f32", 0.0, (5, 20)),
    # causal work order: 2 query tiles and 2 key tiles per head; 32 heads run in
    # windows of 4 heads, 16 K/V heads (dK/dV) in windows of 2
    (2, 16, 16, 200, 200, 128, True, "none", 0.0, None),
    (1, 32, 16, 256, 256, 64, True, "none", 0.0, None),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(i) for i in range(len(BWD_CASES))])
def test_bwd_parity(case):
    B, Hq, Hkv, Lq, Lk, D, causal, bias, softcap, window = case
    print("bwd case", case, flush=True)
    w, q, k, v, do, gkw, okw = make_case(B, Hq, Hkv, Lq, Lk, D, causal, bias, softcap, window)
    got, refs = run_case(w, q, k, v, do, gkw, okw)
    check_grads(got, refs, str(case))


@pytest.mark.parametrize("grad_dtype", [torch.bfloat16, torch.float32])
def test_bwd_grad_dtype(grad_dtype):
    w, q, k, v, do, gkw, okw = make_case(2, 4, 4, 160, 160, 128, True)
    got, refs = run_case(w, q, k, v, do, gkw, okw, grad_dtype)
    assert all(t.dtype == grad_dtype for t in got)
    check_grads(got, refs, "grad dtype %s" % grad_dtype)


@pytest.mark.parametrize("scale", [-0.1, 0.0])
def test_bwd_nonpositive_scale(scale):
    w, q, k, v, do, gkw, okw = make_case(1, 2, 2, 130, 130, 64, True, scale=scale)
    got, refs = run_case(w, q, k, v, do, gkw, okw)
    check_grads(got, refs, "scale %g" % scale)


def test_bwd_oracle_forward_outputs():
    """The backward alone: fed the oracle's O (fp32) and LSE instead of the
    HIP forward's."""
    w, q, k, v, do, gkw, okw = make_case(1, 4, 2, 170, 210, 128, True)
    scale = w.softmax_scale()
    O, L = oracle.attention(q.float(), k.float(), v.float(), scale, True)
    o = torch.from_numpy(O.reshape(1, 4, 170, 128).astype(np.float32)).cuda()
    lse = torch.from_numpy(L.reshape(1, 4, 170).astype(np.float32)).cuda()
    got = attn.attn_bwd(q.cuda(), k.cuda(), v.cuda(), o, lse, do.cuda(), scale, True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(q.float(), k.float(), v.float(), do.float(), scale, True)
    check_grads(got, refs, "oracle O/LSE")


def test_bwd_strided_views():
    """q, k, v, dO as [B, L, H, D] storage viewed as [B, H, L, D]."""
    w, q, k, v, do, gkw, okw = make_case(2, 4, 2, 140, 140, 64, True)
    qs, ks, vs, ds = (t.transpose(1, 2).contiguous().cuda().transpose(1, 2) for t in (q, k, v, do))
    assert not qs.is_contiguous()
    scale = w.softmax_scale()
    o, lse = attn.attn_fwd_prefill(qs, ks, vs, scale, True)
    got = attn.attn_bwd(qs, ks, vs, o, lse, ds, scale, True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(q.float(), k.float(), v.float(), do.float(), scale, True)
    check_grads(got, refs, "strided")


def test_bwd_empty_shapes():
    dev = "cuda"
    q = torch.randn(1, 2, 5, 128, device=dev).to(torch.bfloat16)
    do = torch.randn(1, 2, 5, 128, device=dev).to(torch.bfloat16)
    k0 = torch.empty(1, 1, 0, 128, device=dev, dtype=torch.bfloat16)
    o = torch.zeros(1, 2, 5, 128, device=dev, dtype=torch.bfloat16)
    lse = torch.full((1, 2, 5), -math.inf, device=dev)
    dq = torch.full((1, 2, 5, 128), 7.0, device=dev)
    attn.attn_bwd(q, k0, k0, o, lse, do, None, False, grad_dtype=torch.float32, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)                          # no keys: dq = 0
    q0 = torch.empty(1, 2, 0, 128, device=dev, dtype=torch.bfloat16)
    k = torch.randn(1, 1, 70, 128, device=dev).to(torch.bfloat16)
    dk = torch.full((1, 1, 70, 128), 7.0, device=dev)
    dv = torch.full((1, 1, 70, 128), 7.0, device=dev)
    attn.attn_bwd(q0, k, k, q0, torch.empty(1, 2, 0, device=dev), q0, None, True,
                  grad_dtype=torch.float32, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)   # no rows: dk = dv = 0


def test_bwd_deterministic():
    w, q, k, v, do, gkw, okw = make_case(1, 4, 2, 300, 300, 128, True, "alibi")
    qg, kg, vg, dg = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    scale = w.softmax_scale()
    o, lse = attn.attn_fwd_prefill(qg, kg, vg, scale, True, **gkw)
    a = attn.attn_bwd(qg, kg, vg, o, lse, dg, scale, True, **gkw)
    b = attn.attn_bwd(qg, kg, vg, o, lse, dg, scale, True, **gkw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
