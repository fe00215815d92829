"""Randomised parity sweep: the HIP path against the fp64 oracle over seeded
random combinations of every option (GPU).

Each case draws, from its own seed, the shapes (batch, heads, GQA ratio,
ragged Lq and Lk, including Lq > Lk), head dimension, input and output dtypes,
causal mask, bias kind (none, ALiBi, dense fp32 / bf16 with a broadcast
batch), soft cap and sliding window, and for decode the split count and for
the row L2 norm the row length, split count and output dtype.  The fixed
cases of the other parity tests pin each option on its own; this sweep looks
for interactions between them.  Tolerances are those of the fixed cases.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import online_softmax_fusion_amd as attn

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "bf16": (1.5e-2, 1e-3)}
N_PREFILL, N_DECODE, N_BWD, N_L2 = 48, 32, 20, 16
N_LONG_PREFILL, N_LONG_BWD = 8, 6
N_SPLIT_PREFILL = 16


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


def draw_attention(seed, decode=False, backward=False, long=False):
    rng = np.random.default_rng(seed)
    c = {}
    c["B"] = int(rng.integers(1, 4))
    c["Hkv"] = int(rng.integers(1, 4))
    c["Hq"] = c["Hkv"] * int(rng.choice([1, 2, 3, 4, 5, 8]))   # group sizes that are not powers of two too
    c["D"] = int(rng.choice([64, 128]))
    c["dtype"] = "bf16" if (backward or long or rng.random() < 0.8) else "f32"
    if decode:
        c["Lq"] = int(rng.integers(1, 5))
        c["Lk"] = int(rng.integers(1, 3000))
    elif long and backward:
        c["B"], c["Hkv"], c["Hq"] = 1, 1, int(rng.choice([1, 2]))
        c["Lq"] = int(rng.integers(500, 1200))
        c["Lk"] = int(rng.integers(500, 1200))
    elif long:
        # enough rows and keys per row for the 256-row (eight-wave) workgroup
        c["B"], c["Hkv"] = 1, 1
        c["Hq"] = int(rng.choice([1, 2]))
        c["D"] = 128
        c["Lq"] = int(rng.integers(1024, 1700))
        c["Lk"] = int(rng.integers(4200, 6500))
    else:
        c["Lq"] = int(rng.integers(1, 300))
        c["Lk"] = int(rng.integers(1, 400)) if rng.random() < 0.8 else max(1, c["Lq"] - int(rng.integers(0, 100)))
    c["causal"] = bool(rng.random() < 0.5)
    c["bias"] = str(rng.choice(["none", "none", "alibi", "dense_f32", "dense_bf16"]))
    c["softcap"] = float(rng.choice([0.0, 0.0, 0.0, 3.0, 30.0]))
    c["window"] = None
    if rng.random() < 0.3:
        c["window"] = (int(rng.integers(-1, 120)), int(rng.integers(-1, 60)))
    if long and not backward:   # the eight-wave form takes neither cap nor window
        c["softcap"], c["window"] = 0.0, None
    c["out"] = "f32" if rng.random() < 0.25 else c["dtype"]
    c["splits"] = int(rng.integers(1, 41))
    c["grad"] = "f32" if rng.random() < 0.5 else "bf16"
    # mostly 1/sqrt(D); sometimes a negative, zero or large scale (the kernels
    # fold a positive scale into the exponent and form the score otherwise)
    c["scale"] = None if rng.random() < 0.8 else float(rng.choice([-0.1, 0.0, 0.3, 1.0]))
    c["seed"] = seed
    return c


def make(c):
    w = synth.Workload("random", c["B"], c["Hq"], c["Hkv"], c["Lq"], c["Lk"], c["D"], c["dtype"], c["causal"],
                       c["bias"], c["seed"], scale=c.get("scale"))
    q, k, v = synth.make_qkv(w)
    gkw, okw = {"softcap": c["softcap"], "window": c["window"]}, {"softcap": c["softcap"], "window": c["window"]}
    if c["bias"] == "alibi":
        sl = synth.alibi_slopes(c["Hq"])
        gkw["alibi_slopes"], okw["alibi_slopes"] = sl.cuda(), sl
    elif c["bias"].startswith("dense"):
        bt = synth.make_dense_bias(w, (1, c["Hq"], c["Lq"], c["Lk"]), c["bias"][6:])
        gkw["bias"], okw["bias"] = bt.cuda(), bt.float()
    return w, q, k, v, gkw, okw


def compare(o, lse, O_ref, L_ref, dtype, what, c=None, vmax=None):
    """The fixed cases' bars; where a drawn scale leaves their range, widened
    O by the rounding of the stored output (half an ulp: 2^-8 |O| in bf16,
    2^-24 |O| in fp32; the fixed bars assume |O| below ~3, which peaky rows
    of a large scale exceed), and LSE -- and for fp32 inputs also O, whose
    error is the weights' -- by the score magnitude |scale| sqrt(D) relative
    to the default 1/sqrt(D) (fp32 dot products round in proportion to their
    terms; with bf16 inputs the bf16 rounding of P dominates O).  Given
    vmax = max |v|, a bf16 case may also use the worst-case rounding bound
    2^-9 vmax + half an ulp of |O| (rows that see a few large values of v)."""
    o_tol, l_tol = TOL[dtype]
    half_ulp = 0.0
    if c is not None and c.get("scale") is not None:
        mag = max(1.0, abs(c["scale"]) * c["D"] ** 0.5)
        l_tol *= mag
        if dtype == "f32":
            o_tol *= mag
        half_ulp = 2.0 ** -8 if o.dtype == torch.bfloat16 else 2.0 ** -24
    og = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og)), what + ": non-finite O"
    tol = o_tol + half_ulp * np.abs(O_ref)
    if vmax is not None and dtype == "bf16":
        # the worst case of the rounding: P rounded to bf16 moves each weight
        # by at most 2^-9 of itself, so O by at most 2^-9 max|v|, and the
        # stored output adds half an ulp (2^-8 |O| in bf16, 2^-24 |O| in fp32)
        store = 2.0 ** -8 if o.dtype == torch.bfloat16 else 2.0 ** -24
        tol = np.maximum(tol, 2.0 ** -9 * vmax + store * np.abs(O_ref))
    excess = np.abs(og - O_ref) - tol
    err_o = float(np.max(np.abs(og - O_ref))) if og.size else 0.0
    assert og.size == 0 or float(np.max(excess)) <= 0.0, "%s: O err %.3e" % (what, err_o)
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(lg), fin) and np.all(lg[~fin] == -np.inf), what + ": LSE -inf pattern"
    err_l = float(np.max(np.abs(lg[fin] - L_ref[fin]))) if fin.any() else 0.0
    assert err_l <= l_tol, "%s: LSE err %.3e" % (what, err_l)


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill(i):
    c = draw_attention(6000 + i)
    print("random prefill", c, flush=True)
    w, q, k, v, gkw, okw = make(c)
    od = torch.float32 if c["out"] == "f32" else None
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), c["causal"], out_dtype=od,
                                   **gkw)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), c["causal"], **okw)
    compare(o, lse, O_ref, L_ref, c["dtype"], str(c), c, vmax=float(v.float().abs().max()))
    # the automatically planned forward gives the same result within the same bars
    o2, lse2 = attn.attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), c["causal"], out_dtype=od, **gkw)
    torch.cuda.synchronize()
    compare(o2, lse2, O_ref, L_ref, c["dtype"], "attn_fwd " + str(c), c, vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("i", range(N_LONG_PREFILL))
def test_random_long_prefill(i):
    """Shapes that run the 256-row (eight-wave) workgroup, sampled rows."""
    c = draw_attention(6500 + i, long=True)
    print("random long prefill", c, flush=True)
    w, q, k, v, gkw, okw = make(c)
    od = torch.float32 if c["out"] == "f32" else None
    o, lse = attn.attn_fwd_prefill(q.cuda(), k.cuda(), v.cuda(), w.softmax_scale(), c["causal"], out_dtype=od,
                                   **gkw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(c["seed"])
    n = c["B"] * c["Hq"] * c["Lq"]
    rows = np.unique(np.concatenate([np.arange(0, 300), np.arange(n - 300, n), rng.integers(0, n, 200)]))
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), c["causal"], rows=rows, **okw)
    compare(o.reshape(n, -1)[rows], lse.reshape(n)[rows], O_ref, L_ref, c["dtype"], str(c), c)


@pytest.mark.parametrize("i", range(N_SPLIT_PREFILL))
def test_random_split_prefill(i):
    """The prefill kernel over key chunks and the combine (bf16 inputs), with
    1 to 8 chunks of whole 64-key tiles over up to 3000 keys (so chunks past
    the keys, and chunks a row cannot see, occur)."""
    c = draw_attention(9000 + i)
    rng = np.random.default_rng(90000 + i)
    c["dtype"] = "bf16"
    c["out"] = "f32" if c["out"] == "f32" else "bf16"
    c["Lk"] = int(rng.integers(1, 3000))
    c["splits"] = int(rng.integers(1, 9))
    print("random split prefill", c, flush=True)
    w, q, k, v, gkw, okw = make(c)
    od = torch.float32 if c["out"] == "f32" else torch.bfloat16
    op, mp, lp = attn.attn_fwd_prefill_splitk(q.cuda(), k.cuda(), v.cuda(), c["splits"], w.softmax_scale(),
                                              c["causal"], **gkw)
    o, lse = attn.attn_splitk_combine(op, mp, lp, out_dtype=od)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), c["causal"], **okw)
    compare(o, lse, O_ref, L_ref, c["dtype"], str(c), c, vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode(i):
    c = draw_attention(7000 + i, decode=True)
    print("random decode", c, flush=True)
    w, q, k, v, gkw, okw = make(c)
    od = torch.float32 if c["out"] == "f32" else q.dtype
    o, lse = attn.decode(q.cuda(), k.cuda(), v.cuda(), c["splits"], w.softmax_scale(), c["causal"], out_dtype=od,
                         **gkw)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), c["causal"], **okw)
    compare(o, lse, O_ref, L_ref, c["dtype"], str(c), c, vmax=float(v.float().abs().max()))


@pytest.mark.parametrize("i", range(N_BWD + N_LONG_BWD))
def test_random_backward(i):
    """Gradients under the bars of the backward parity tests (max |err| <=
    2e-2 max |ref|, relative Frobenius error <= 8e-3 per tensor); the last
    cases span many query and key tiles."""
    c = draw_attention(8000 + i, backward=True, long=i >= N_BWD)
    print("random backward", c, flush=True)
    w, q, k, v, gkw, okw = make(c)
    do = synth.make_dout(w)
    s = w.softmax_scale()
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o, lse = attn.attn_fwd_prefill(qc, kc, vc, s, c["causal"], **gkw)
    gd = torch.float32 if c["grad"] == "f32" else torch.bfloat16
    got = attn.attn_bwd(qc, kc, vc, o, lse, do.cuda(), s, c["causal"], grad_dtype=gd, **gkw)
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(q, k, v, do, s, c["causal"], **okw)
    # a gradient that vanishes in exact arithmetic (e.g. dQ when every row sees
    # one key: dS = dP - Delta = 0) carries only rounding: bound it by the
    # problem's gradient scale
    gscale = max([float(np.max(np.abs(r))) for r in refs if r.size] + [0.0])
    for name, g, ref in zip(("dq", "dk", "dv"), got, refs):
        gg = g.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(gg)), name
        scale = float(np.max(np.abs(ref))) if ref.size else 0.0
        if scale == 0.0:
            if gg.size:
                assert float(np.max(np.abs(gg))) <= 2e-2 * gscale, "%s %s must vanish" % (c, name)
            continue
        err = np.abs(gg - ref)
        mx = float(np.max(err)) / scale
        fro = float(np.linalg.norm(err) / np.linalg.norm(ref))
        assert mx <= 2e-2 and fro <= 8e-3, "%s %s: max %.3e fro %.3e" % (c, name, mx, fro)


@pytest.mark.parametrize("i", range(N_L2))
def test_random_l2norm(i):
    rng = np.random.default_rng(9000 + i)
    dt = "bf16" if rng.random() < 0.5 else "f32"
    vec = 8 if dt == "bf16" else 4
    rows = int(rng.integers(1, 50))
    H = vec * int(rng.integers(1, 20000 // vec))
    maxone = attn.l2norm_max_onepass(synth.torch_dtype(dt))
    S = int(rng.integers(2, 10)) if (H > maxone or rng.random() < 0.5) else 1
    out_dt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    print("random l2norm", rows, H, dt, S, out_dt, flush=True)
    x = synth.make_rows(synth.RowsWorkload("random", rows, H, dt, 9000 + i))
    y, n = attn.l2norm_rows(x.cuda(), out_dtype=out_dt, num_splits=S)
    torch.cuda.synchronize()
    Y, N = oracle.l2norm(x.float())
    assert float(np.max(np.abs(n.cpu().double().numpy() - N) / N)) <= 1e-5
    tol = (2.0 ** -8 if out_dt == torch.bfloat16 else 2.0 ** -23) + 1e-5
    yg = y.float().cpu().double().numpy()
    assert np.all(np.abs(yg - Y) <= tol * np.abs(Y) + 1e-37)
