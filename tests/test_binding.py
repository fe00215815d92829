"""Argument checks of the Python binding (CPU, plus GPU cases).

The binding passes raw pointers to the C ABI, which cannot tell a host
pointer, a buffer of the wrong size or a buffer on another device from a good
one.  Every entry point must therefore refuse such tensors before anything
is enqueued.  The CPU cases check that host tensors are refused without a
launch; the GPU cases check output shapes, LSE and norm buffers, and that a
non-contiguous slopes vector (copied inside the binding) gives the same
result as a contiguous one.
"""
import pytest
import torch

import synth
import online_softmax_fusion_amd as attn


def _cpu_qkv():
    w = synth.Workload(name="binding", B=1, Hq=2, Hkv=1, Lq=40, Lk=70, D=64, dtype="bf16", seed=4001)
    return synth.make_qkv(w)


def test_host_tensors_are_refused():
    q, k, v = _cpu_qkv()
    with pytest.raises(ValueError, match="GPU"):
        attn.attn_fwd_prefill(q, k, v)
    with pytest.raises(ValueError, match="GPU"):
        attn.attn_fwd(q, k, v)
    with pytest.raises(ValueError, match="GPU"):
        attn.attn_fwd_decode_splitk(q, k, v, 2)
    with pytest.raises(ValueError, match="GPU"):
        attn.decode(q, k, v, 2)
    with pytest.raises(ValueError, match="GPU"):
        attn.l2norm_rows(torch.ones(4, 64))
    o = torch.empty(1, 2, 40, 64, dtype=torch.bfloat16)
    lse = torch.empty(1, 2, 40)
    with pytest.raises(ValueError, match="GPU"):
        attn.attn_bwd(q, k, v, o, lse, o)
    parts = torch.empty(1, 2, 1, 3, 64), torch.empty(1, 2, 1, 3), torch.empty(1, 2, 1, 3)
    with pytest.raises(ValueError, match="GPU"):
        attn.attn_splitk_combine(*parts)


gpu = pytest.mark.gpu


def _gpu_qkv():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return [t.cuda() for t in _cpu_qkv()]


@gpu
def test_mixed_host_and_device_tensors_are_refused():
    q, k, v = _gpu_qkv()
    with pytest.raises(ValueError, match="k must be"):
        attn.attn_fwd_prefill(q, k.cpu(), v)
    with pytest.raises(ValueError, match="bias must be on"):
        attn.attn_fwd_prefill(q, k, v, bias=torch.zeros(40, 70))
    with pytest.raises(ValueError, match="alibi_slopes must be on"):
        attn.attn_fwd_prefill(q, k, v, alibi_slopes=torch.ones(2))
    with pytest.raises(ValueError, match="lse must be on"):
        attn.attn_fwd_prefill(q, k, v, lse=torch.empty(1, 2, 40))


@gpu
def test_wrong_output_buffers_are_refused():
    q, k, v = _gpu_qkv()
    small = torch.empty(1, 2, 39, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out must be"):
        attn.attn_fwd_prefill(q, k, v, out=small)
    with pytest.raises(ValueError, match="out must be"):
        attn.attn_fwd(q, k, v, out=small)
    with pytest.raises(ValueError, match="lse must be"):
        attn.attn_fwd_prefill(q, k, v, lse=torch.empty(1, 2, 39, device="cuda"))
    with pytest.raises(ValueError, match="lse must be"):
        attn.attn_fwd(q, k, v, lse=torch.empty(80, device="cuda", dtype=torch.float64))
    o_part, m_part, l_part = attn.attn_fwd_decode_splitk(q, k, v, 3)
    with pytest.raises(ValueError, match="out must be"):
        attn.attn_splitk_combine(o_part, m_part, l_part, out=small)
    with pytest.raises(ValueError, match="lse must be"):
        attn.attn_splitk_combine(o_part, m_part, l_part, lse=torch.empty(1, 2, 41, device="cuda"))
    o, lse = attn.attn_fwd_prefill(q, k, v)
    with pytest.raises(ValueError, match="dq must be"):
        attn.attn_bwd(q, k, v, o, lse, o, dq=small)
    with pytest.raises(ValueError, match="o must be"):
        attn.attn_bwd(q, k, v, small, lse, o)
    x = torch.ones(4, 64, device="cuda")
    with pytest.raises(ValueError, match="norm must be"):
        attn.l2norm_rows(x, norm=torch.empty(3, device="cuda"))
    torch.cuda.synchronize()


@gpu
def test_strided_slopes_match_contiguous():
    """ALiBi slopes given as a strided view are copied by the binding; the
    copy lives until the launch has read it, and the result is bitwise the
    contiguous one's (prefill, decode, backward)."""
    q, k, v = _gpu_qkv()
    s = synth.alibi_slopes(2).cuda()
    wide = torch.zeros(4, device="cuda")
    wide[::2] = s
    strided = wide[::2]
    assert not strided.is_contiguous()
    o1, l1 = attn.attn_fwd_prefill(q, k, v, 0.125, True, alibi_slopes=s)
    o2, l2 = attn.attn_fwd_prefill(q, k, v, 0.125, True, alibi_slopes=strided)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    d1, e1 = attn.decode(q, k, v, 3, 0.125, alibi_slopes=s)
    d2, e2 = attn.decode(q, k, v, 3, 0.125, alibi_slopes=strided)
    assert torch.equal(d1, d2) and torch.equal(e1, e2)
    g1 = attn.attn_bwd(q, k, v, o1, l1, o1, 0.125, True, alibi_slopes=s)
    g2 = attn.attn_bwd(q, k, v, o1, l1, o1, 0.125, True, alibi_slopes=strided)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
