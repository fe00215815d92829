"""Addresses beyond 4 GiB (GPU).

Every tensor of these cases is a strided view whose batch (or row) stride is
2^31 elements, so the second batch's data sits more than 4 GiB (bf16) or
8 GiB (fp32) past the base pointer and every element offset of it exceeds
the 32-bit range.  Only the viewed elements are written or read; the gaps are
never touched.  Each view needs one allocation of 2^31 elements plus a head,
4-8 GiB, freed after the case.  Results are compared with the fp64 oracle
under the tolerances of the small-size parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import online_softmax_fusion_amd as attn

pytestmark = pytest.mark.gpu

FAR = 2 ** 31          # elements between the two batches (or rows) of every view


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


@pytest.fixture(autouse=True)
def free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def far_view(shape, dtype, src=None):
    """A [2, ...] view with batch stride FAR over one allocation; the inner
    dimensions are contiguous.  Filled from ``src`` (same shape) if given."""
    assert shape[0] == 2
    inner = int(np.prod(shape[1:]))
    store = torch.empty(FAR + inner, dtype=dtype, device="cuda")
    strides = [FAR] + [int(np.prod(shape[i + 1:])) for i in range(1, len(shape))]
    t = store.as_strided(tuple(shape), tuple(strides))
    if src is not None:
        t.copy_(src)
    return t


def workload(B, Hq, Hkv, Lq, Lk, D, dtype, seed):
    return synth.Workload(name="far-offsets", B=B, Hq=Hq, Hkv=Hkv, Lq=Lq, Lk=Lk, D=D, dtype=dtype, seed=seed)


def qkv(B, Hq, Hkv, Lq, Lk, D, dtype, seed):
    return synth.make_qkv(workload(B, Hq, Hkv, Lq, Lk, D, dtype, seed))


def check(o, lse, O_ref, L_ref, o_tol, lse_tol, what):
    eo = float(np.max(np.abs(o.float().cpu().double().numpy() - O_ref)))
    el = float(np.max(np.abs(lse.cpu().double().numpy() - L_ref)))
    print("%s: O err %.3e, LSE err %.3e" % (what, eo, el), flush=True)
    assert eo <= o_tol and el <= lse_tol, what


@pytest.mark.parametrize("causal,bias", [(True, "none"), (False, "dense_bf16"), (True, "alibi")])
def test_prefill_far_offsets(causal, bias):
    """bf16 prefill, GQA 2:1, ragged Lq = 200 against Lk = 300; q, k, v, O
    (and a dense bias) at batch stride 2^31 elements."""
    print("far-offset prefill", causal, bias, flush=True)
    B, Hq, Hkv, Lq, Lk, D = 2, 2, 1, 200, 300, 128
    q, k, v = qkv(B, Hq, Hkv, Lq, Lk, D, "bf16", 3001)
    scale = D ** -0.5
    qg, kg, vg = (far_view(t.shape, torch.bfloat16, t.cuda()) for t in (q, k, v))
    og = far_view((B, Hq, Lq, D), torch.bfloat16)
    kw, ref_kw = {}, {}
    if bias == "dense_bf16":
        bb = synth.make_dense_bias(workload(B, Hq, Hkv, Lq, Lk, D, "bf16", 3002), (B, Hq, Lq, Lk), "bf16")
        kw["bias"] = far_view(bb.shape, torch.bfloat16, bb.cuda())
        ref_kw["bias"] = bb.float()
    elif bias == "alibi":
        s = synth.alibi_slopes(Hq)
        kw["alibi_slopes"] = s.cuda()
        ref_kw["alibi_slopes"] = s
    o, lse = attn.attn_fwd_prefill(qg, kg, vg, scale, causal, out=og, **kw)
    torch.cuda.synchronize()
    assert o.data_ptr() == og.data_ptr()
    O_ref, L_ref = oracle.attention(q.float(), k.float(), v.float(), scale, causal, **ref_kw)
    check(o, lse, O_ref, L_ref, 1.5e-2, 1e-3, "prefill causal=%s bias=%s" % (causal, bias))


def test_prefill_f32_far_offsets():
    """fp32 path (vector ALU kernel), d = 64, batch stride 2^31 fp32 elements
    (8 GiB)."""
    print("far-offset fp32 prefill", flush=True)
    B, H, L, D = 2, 1, 96, 64
    q, k, v = qkv(B, H, H, L, L, D, "f32", 3003)
    qg, kg, vg = (far_view(t.shape, torch.float32, t.cuda()) for t in (q, k, v))
    og = far_view((B, H, L, D), torch.float32)
    o, lse = attn.attn_fwd_prefill(qg, kg, vg, 0.125, True, out=og)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q, k, v, 0.125, True)
    check(o, lse, O_ref, L_ref, 1e-5, 1e-5, "fp32 prefill")


def test_decode_far_offsets():
    """Split-K decode (GQA 4:1, Lk = 5000 ragged over the chunks) with K and V
    at batch stride 2^31 elements, and the combine writing O at the same
    stride."""
    print("far-offset decode", flush=True)
    B, Hq, Hkv, Lk, D = 2, 8, 2, 5000, 128
    q, k, v = qkv(B, Hq, Hkv, 1, Lk, D, "bf16", 3004)
    scale = D ** -0.5
    kg, vg = (far_view(t.shape, torch.bfloat16, t.cuda()) for t in (k, v))
    og = far_view((B, Hq, 1, D), torch.bfloat16)
    o, lse = attn.decode(q.cuda(), kg, vg, 7, scale, out=og)
    torch.cuda.synchronize()
    assert o.data_ptr() == og.data_ptr()
    O_ref, L_ref = oracle.attention(q.float(), k.float(), v.float(), scale, False)
    check(o, lse, O_ref, L_ref, 1.5e-2, 1e-3, "decode")


def test_backward_far_offsets():
    """attn_bwd (causal, L = 260 ragged) with q, k, v, O, dO, dQ, dK, dV all at
    batch stride 2^31 elements; the bars of the backward parity tests."""
    print("far-offset backward", flush=True)
    B, H, L, D = 2, 1, 260, 128
    q, k, v = qkv(B, H, H, L, L, D, "bf16", 3005)
    do = synth.make_dout(workload(B, H, H, L, L, D, "bf16", 3006))
    scale = D ** -0.5
    qg, kg, vg, dog = (far_view(t.shape, torch.bfloat16, t.cuda()) for t in (q, k, v, do))
    og = far_view((B, H, L, D), torch.bfloat16)
    _, lse = attn.attn_fwd_prefill(qg, kg, vg, scale, True, out=og)
    grads = [far_view((B, H, L, D), torch.float32) for _ in range(3)]
    dq, dk, dv = attn.attn_bwd(qg, kg, vg, og, lse, dog, scale, True, grad_dtype=torch.float32,
                               dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    refs = oracle.attention_bwd(q.float(), k.float(), v.float(), do.float(), scale, True)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        g = got.cpu().double().numpy()
        for b in range(B):
            err = np.abs(g[b] - ref[b])
            mx = float(np.max(err)) / float(np.max(np.abs(ref[b])))
            fro = float(np.linalg.norm(err) / np.linalg.norm(ref[b]))
            print("backward %s b=%d: max %.3e fro %.3e" % (name, b, mx, fro), flush=True)
            assert mx <= 2e-2 and fro <= 8e-3, (name, b)


@pytest.mark.parametrize("splits", [1, 3])
def test_l2norm_far_offsets(splits):
    """Row L2 norm of 2 rows of 4096 bf16 elements that lie 2^31 elements
    apart, y written at the same row stride; one pass and split-K."""
    print("far-offset l2norm splits=%d" % splits, flush=True)
    w = synth.RowsWorkload(name="far-offsets-rows", rows=2, H=4096, dtype="bf16", seed=3007)
    x = synth.make_rows(w)
    xs = torch.empty(FAR + 4096, dtype=torch.bfloat16, device="cuda").as_strided((2, 4096), (FAR, 1))
    xs.copy_(x.cuda())
    ys = torch.empty(FAR + 4096, dtype=torch.bfloat16, device="cuda").as_strided((2, 4096), (FAR, 1))
    y, n = attn.l2norm_rows(xs, out=ys, num_splits=splits)
    torch.cuda.synchronize()
    Y, N = oracle.l2norm(x.float())
    assert float(np.max(np.abs(n.cpu().double().numpy() - N) / N)) <= 1e-5
    yg = y.float().cpu().double().numpy()
    assert np.all(np.abs(yg - Y) <= (2.0 ** -8 + 1e-5) * np.abs(Y) + 1e-37)
