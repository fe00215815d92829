"""Parity at the full workload sizes, in the launch configuration bench.py
times, on sampled output rows that the fp64 oracle computes one by one (GPU).

Inputs are drawn on the GPU with the seeded recipe of ``synth``; the oracle
receives host copies of exactly the stored values of the heads it needs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import online_softmax_fusion_amd as attn

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 1.5e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


def sample_rows(L, rng, n=10):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, L // 2, L - 129, L - 128, L - 2, L - 1]
    rnd = rng.integers(0, L, size=n).tolist()
    return sorted({r for r in fixed + rnd if 0 <= r < L})


def check_heads(w, q, k, v, o, lse, heads, rows, slopes=None, bias=None):
    """Compare rows of heads [(b, h), ...] against the oracle, per head
    (rows=None: every row of the head).  ``bias``: a dense [Hq, Lq, Lk] bias
    on the GPU, broadcast over the batch."""
    G = w.Hq // w.Hkv
    worst_o = worst_l = 0.0
    for b, h in heads:
        hk = h // G
        qh = q[b:b + 1, h:h + 1].float().cpu()
        kh = k[b:b + 1, hk:hk + 1].float().cpu()
        vh = v[b:b + 1, hk:hk + 1].float().cpu()
        kw = {}
        if slopes is not None:
            kw["alibi_slopes"] = slopes[h:h + 1]
        if bias is not None:
            kw["bias"] = bias[h:h + 1].float().cpu()
        O_ref, L_ref = oracle.attention(qh, kh, vh, w.softmax_scale(), w.causal, rows=rows, softcap=w.softcap,
                                        window=w.window, **kw)
        sel = slice(None) if rows is None else rows
        og = o[b, h, sel].float().cpu().numpy()
        lg = lse[b, h, sel].cpu().numpy()
        O_ref, L_ref = O_ref.reshape(og.shape), L_ref.reshape(lg.shape)
        eo = float(np.max(np.abs(og - O_ref)))
        el = float(np.max(np.abs(lg - L_ref)))
        assert eo <= O_TOL, "%s b=%d h=%d: O err %.3e" % (w.name, b, h, eo)
        assert el <= LSE_TOL, "%s b=%d h=%d: LSE err %.3e" % (w.name, b, h, el)
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    print("%s: worst O err %.3e, worst LSE err %.3e" % (w.name, worst_o, worst_l), flush=True)


@pytest.mark.parametrize("w", [synth.C2_CAUSAL, synth.C3_ALIBI, synth.C5_PREFILL, synth.SOFTCAP_PREFILL,
                               synth.WINDOW_PREFILL], ids=lambda w: w.name)
def test_prefill_fullsize_sampled(w):
    print("full-size prefill", w.name, flush=True)
    rng = np.random.default_rng(w.seed)
    q, k, v = synth.make_qkv(w, device="cuda")
    slopes = synth.alibi_slopes(w.Hq) if w.bias == "alibi" else None
    kw = {"alibi_slopes": slopes.cuda()} if slopes is not None else {}
    o, lse = attn.attn_fwd_prefill(q, k, v, w.softmax_scale(), w.causal, softcap=w.softcap, window=w.window, **kw)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    heads = sorted({(0, 0), (w.B - 1, w.Hq - 1), (w.B // 2, w.Hq // 2)} |
                   {(int(rng.integers(w.B)), int(rng.integers(w.Hq))) for _ in range(2)})
    check_heads(w, q, k, v, o, lse, heads, sample_rows(w.Lq, rng), slopes)


@pytest.mark.parametrize("w", [synth.C2_CAUSAL, synth.C3_ALIBI], ids=lambda w: w.name)
def test_prefill_fullsize_whole_heads(w):
    """Two heads of the full-size launch compared in full: every row and
    every column of O and every LSE, against the oracle over the whole head."""
    print("full-size prefill, whole heads", w.name, flush=True)
    q, k, v = synth.make_qkv(w, device="cuda")
    slopes = synth.alibi_slopes(w.Hq) if w.bias == "alibi" else None
    kw = {"alibi_slopes": slopes.cuda()} if slopes is not None else {}
    o, lse = attn.attn_fwd_prefill(q, k, v, w.softmax_scale(), w.causal, **kw)
    torch.cuda.synchronize()
    check_heads(w, q, k, v, o, lse, [(0, 0), (w.B - 1, w.Hq - 1)], None, slopes)


def test_prefill_fullsize_dense_bias():
    """The ALiBi causal workload with its bias given as a bf16 [H, L, L]
    tensor broadcast over the batch (the form bench.py times): sampled rows of
    five heads, and one head in full, against the oracle on the same stored
    bias values."""
    w = synth.C3_DENSE
    print("full-size prefill, dense bias", w.name, flush=True)
    rng = np.random.default_rng(w.seed + 1)
    q, k, v = synth.make_qkv(w, device="cuda")
    bias = synth.alibi_bias_tensor(w, "bf16", "cuda")
    o, lse = attn.attn_fwd_prefill(q, k, v, w.softmax_scale(), w.causal, bias=bias)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    heads = sorted({(0, 0), (w.B - 1, w.Hq - 1), (w.B // 2, w.Hq // 2)} |
                   {(int(rng.integers(w.B)), int(rng.integers(w.Hq))) for _ in range(2)})
    check_heads(w, q, k, v, o, lse, heads, sample_rows(w.Lq, rng), bias=bias)
    check_heads(w, q, k, v, o, lse, [(1, 3)], None, bias=bias)


@pytest.mark.parametrize("w", [synth.C4_DECODE, synth.C5_DECODE], ids=lambda w: w.name)
def test_decode_fullsize(w):
    print("full-size decode", w.name, flush=True)
    q, k, v = synth.make_qkv(w, device="cuda")
    S = w.splits or attn.attn_decode_choose_splits(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, attn.attn_device_cu_count(0))
    o, lse = attn.decode(q, k, v, S, w.softmax_scale())
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(w.seed)
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    if len(heads) > 64:
        idx = rng.choice(len(heads), size=64, replace=False)
        heads = sorted(heads[i] for i in idx)
    check_heads(w, q, k, v, o, lse, heads, [0])


def test_tiny_reference_workload():
    """The fp32 L=256, d=64 workload in full, 1e-5 on O and LSE."""
    w = synth.C1_TINY
    q, k, v = synth.make_qkv(w)
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), w.causal)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), w.causal)
    assert float(np.max(np.abs(o.cpu().double().numpy() - O_ref))) <= 1e-5
    assert float(np.max(np.abs(lse.cpu().double().numpy() - L_ref))) <= 1e-5


@pytest.mark.parametrize("w", [synth.BWD_PREFILL, synth.C2_CAUSAL], ids=lambda w: w.name)
def test_backward_fullsize_sampled_heads(w):
    """attn_bwd on the whole workload (bf16 gradients, as bench.py times it);
    four (b, h) heads compared in full (every row of dQ, every key of dK, dV)
    with the oracle's gradients of those heads, under the tolerances of the
    small-size backward tests (max |err| <= 2e-2 * max |ref|, relative
    Frobenius error <= 8e-3)."""
    print("full-size backward", w.name, flush=True)
    assert w.Hq == w.Hkv
    q, k, v = synth.make_qkv(w, device="cuda")
    do = synth.make_dout(w, device="cuda")
    scale = w.softmax_scale()
    o, lse = attn.attn_fwd_prefill(q, k, v, scale, w.causal)
    dq, dk, dv = attn.attn_bwd(q, k, v, o, lse, do, scale, w.causal)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    rng = np.random.default_rng(w.seed)
    heads = [(0, 0), (w.B - 1, w.Hq - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.Hq))) for _ in range(2)]
    # the heads are independent: stack them as a batch of one-head problems
    pick = lambda t: torch.stack([t[b, h] for b, h in heads]).unsqueeze(1).float().cpu()
    refs = oracle.attention_bwd(pick(q), pick(k), pick(v), pick(do), scale, w.causal, threads=len(heads))
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g = pick(got).numpy().astype(np.float64)
        for n, (b, h) in enumerate(heads):
            scale_ref = float(np.max(np.abs(ref[n])))
            err = np.abs(g[n] - ref[n])
            mx = float(np.max(err)) / scale_ref
            fro = float(np.linalg.norm(err) / np.linalg.norm(ref[n]))
            assert mx <= 2e-2 and fro <= 8e-3, "%s %s b=%d h=%d: max %.3e fro %.3e" % (w.name, name, b, h, mx, fro)
        print("%s %s: max|err|/max|ref| <= %.2e" % (w.name, name, max(
            float(np.max(np.abs(g[n] - ref[n]))) / float(np.max(np.abs(ref[n]))) for n in range(len(heads)))),
            flush=True)


@pytest.mark.parametrize("w", [synth.L2N_ROWS, synth.L2N_LONG], ids=lambda w: w.name)
def test_l2norm_fullsize(w):
    """The row L2 norm workloads in the configuration bench.py times (split
    count from l2norm_choose_splits), norms of every row and sampled rows of
    y against the oracle, under the tolerances of tests/test_l2norm_gpu.py."""
    print("full-size l2norm", w.name, flush=True)
    x = synth.make_rows(w, device="cuda")
    S = attn.l2norm_choose_splits(w.rows, w.H, x.dtype, attn.attn_device_cu_count(0))
    y, n = attn.l2norm_rows(x, num_splits=S)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed)
    rows = sorted(set([0, 1, w.rows - 1] + rng.integers(0, w.rows, size=min(w.rows, 64)).tolist()))
    xs = x[rows].float().cpu()
    Y, N = oracle.l2norm(xs)
    ng = n[rows].double().cpu().numpy()
    assert float(np.max(np.abs(ng - N) / N)) <= 1e-5
    yg = y[rows].float().cpu().double().numpy()
    tol = 2.0 ** -8 + 1e-5 if x.dtype == torch.bfloat16 else 1e-5 + 2.0 ** -24
    assert np.all(np.abs(yg - Y) <= tol * np.abs(Y) + 1e-37)
    print("%s: S=%d, worst norm rel err %.2e" % (w.name, S, float(np.max(np.abs(ng - N) / N))), flush=True)
