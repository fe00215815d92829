"""Row L2 norm (l2norm_rows) against the fp64 oracle (GPU), one pass and
split-K, through the C ABI.

Tolerances.  norm: relative error <= 1e-5.  Every square is scaled by an
exact power of two and the sums are of non-negative terms, so the relative
error is at most (terms per sequential chain + merge levels) * 2^-24: at
most 128 terms per lane plus 8 levels of merging, 8.1e-6.  y: relative error
<= 1e-5 + 2^-24 with fp32 output, <= 2^-8 + 1e-5 with bf16 output (the
round-to-nearest of bf16 adds at most 2^-9 relative)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import online_softmax_fusion_amd as attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


def make_rows(rows, H, dtype, seed, scales=None):
    x = synth.normal((rows, H), seed, 0, "f32")
    if scales is not None:
        x = x * torch.tensor(scales, dtype=torch.float32)[:, None]
    return x.to(synth.torch_dtype(dtype))


def check(x, y, n, out_dtype, what=""):
    Y, N = oracle.l2norm(x.float())
    ng = n.cpu().double().numpy()
    nz = N > 0
    assert np.all(ng[~nz] == 0.0), what + ": zero rows must have norm 0"
    rel = np.abs(ng[nz] - N[nz]) / N[nz]
    assert rel.size == 0 or float(rel.max()) <= 1e-5, "%s: norm rel err %.3e" % (what, float(rel.max()))
    if y is not None:
        yg = y.float().cpu().double().numpy()
        tol = 2.0 ** -8 + 1e-5 if out_dtype == torch.bfloat16 else 1e-5 + 2.0 ** -24
        err = np.abs(yg - Y)
        assert np.all(err <= tol * np.abs(Y) + 1e-37), "%s: y rel err %.3e" % (
            what, float(np.max(err / np.maximum(np.abs(Y), 1e-37))))
        assert np.all(yg[~nz] == 0.0)
    return float(rel.max()) if rel.size else 0.0


CASES = [
    # rows, H, x dtype, y dtype, splits (None: chosen)
    (37, 8, "bf16", torch.bfloat16, None),
    (37, 1000, "bf16", torch.bfloat16, None),
    (129, 4096, "bf16", torch.bfloat16, None),
    (5, 8192, "bf16", torch.float32, None),        # widest one-pass row
    (33, 4, "f32", torch.float32, None),
    (33, 1004, "f32", torch.bfloat16, None),
    (9, 4096, "f32", torch.float32, None),
    (3, 100000, "bf16", torch.bfloat16, None),     # split-K
    (2, 300000, "f32", torch.float32, None),
    (4, 4096, "bf16", torch.bfloat16, 3),           # split-K by request on a short row
    (4, 40000, "f32", torch.float32, 1000),        # more chunks than some rows need: empty chunks
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_l2norm_parity(case):
    rows, H, dt, ydt, S = case
    print("l2norm case", case, flush=True)
    x = make_rows(rows, H, dt, 31)
    y, n = attn.l2norm_rows(x.cuda(), out_dtype=ydt, num_splits=S)
    torch.cuda.synchronize()
    check(x, y, n, ydt, str(case))


@pytest.mark.parametrize("splits", [1, 6])
def test_l2norm_extreme_magnitudes(splits):
    """Rows whose plain fp32 sum of squares would overflow (entries ~1e36:
    squares ~1e72, norm ~6e37 still in range) or underflow (1e-30, and
    denormals near 1e-37 and 1e-45), zero and one-hot rows, all in one
    launch."""
    H = 4096
    x = make_rows(8, H, "f32", 32, [1e36, 1e30, 1.0, 1e-30, 1e-37, 1.0, 0.0, 0.0])
    x[5] = 0.0
    x[5, 17] = -2.5
    x[7, H - 1] = 1e-45                                   # a single denormal
    y, n = attn.l2norm_rows(x.cuda(), out_dtype=torch.float32, num_splits=splits)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(n).all())
    check(x, y, n, torch.float32, "extreme, splits %d" % splits)
    assert float(n[5]) == 2.5 and float(y[5, 17]) == -1.0


def test_l2norm_strided_rows_and_norm_only():
    base = make_rows(6, 3072, "bf16", 33)
    x = base.cuda()[:, 1024:]                 # rows 3072 apart, 2048 long
    assert x.stride(0) == 3072
    y, n = attn.l2norm_rows(x)
    _, n2 = attn.l2norm_rows(x, return_y=False)
    torch.cuda.synchronize()
    check(base[:, 1024:].contiguous(), y, n, torch.bfloat16, "strided")
    assert torch.equal(n, n2)


def test_l2norm_onepass_equals_split():
    x = make_rows(16, 8192, "bf16", 34).cuda()
    y1, n1 = attn.l2norm_rows(x, num_splits=1, out_dtype=torch.float32)
    y2, n2 = attn.l2norm_rows(x, num_splits=8, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert float(((n1 - n2).abs() / n1).max()) <= 2e-6
    assert float((y1 - y2).abs().max()) <= 2e-6
