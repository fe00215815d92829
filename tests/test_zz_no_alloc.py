"""attn_fwd_noalloc (the planned forward with its partials in the library's
fixed per-device array) against attn_fwd with a caller workspace, through the
C ABI (GPU).  Two calls in a row on split plans, the second smaller than the
first, each compared with attn_fwd at the bf16 bars of the other forward
tests (1.5e-2 on O, 1e-3 on LSE); the second also against the fp64 oracle.
A plan whose partials exceed the array is rejected before anything is
enqueued."""
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


def _inputs(B, Hq, Hkv, Lq, Lk, causal, seed):
    w = synth.Workload("noalloc", B, Hq, Hkv, Lq, Lk, 128, "bf16", causal, "none", seed)
    q, k, v = synth.make_qkv(w)
    return w, q, k, v


def _noalloc(qg, kg, vg, w):
    B, Hq, Lq, D = qg.shape
    out = torch.full((B, Hq, Lq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device="cuda")
    return attn.attn_fwd_noalloc(qg, kg, vg, w.softmax_scale(), w.causal, out=out, lse=lse)


def _close(o1, l1, o2, l2):
    assert bool(torch.isfinite(o1.float()).all())
    assert float((o1.float() - o2.float()).abs().max()) <= 1.5e-2
    fin = torch.isfinite(l2)
    assert torch.equal(torch.isfinite(l1), fin)
    if bool(fin.any()):
        assert float((l1[fin] - l2[fin]).abs().max()) <= 1e-3


# B, Hq, Hkv, Lq, Lk, causal, plan: a large split prefill, then a smaller split-K;
# a large split-K, then a smaller split prefill
SEQUENCES = [
    [(1, 8, 8, 2048, 32768, True, attn.ATTN_PLAN_PREFILL_SPLIT), (1, 8, 2, 1, 3000, False, attn.ATTN_PLAN_SPLITK)],
    [(4, 32, 8, 1, 8192, False, attn.ATTN_PLAN_SPLITK), (1, 32, 8, 100, 3000, True, attn.ATTN_PLAN_PREFILL_SPLIT)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["prefill_split_then_splitk", "splitk_then_prefill_split"])
def test_noalloc_matches_attn_fwd_twice(seq):
    for i, (B, Hq, Hkv, Lq, Lk, causal, want) in enumerate(seq):
        print("attn_fwd_noalloc call", i, (B, Hq, Hkv, Lq, Lk, causal), flush=True)
        w, q, k, v = _inputs(B, Hq, Hkv, Lq, Lk, causal, 31 + i)
        qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
        plan = attn.attn_fwd_choose_plan(qg, kg, vg, w.softmax_scale(), causal)
        assert plan.method == want
        assert 0 < plan.workspace_bytes <= attn.NOALLOC_SCRATCH_BYTES
        o_na, l_na = _noalloc(qg, kg, vg, w)
        o_ws, l_ws = attn.attn_fwd(qg, kg, vg, w.softmax_scale(), causal)
        torch.cuda.synchronize()
        _close(o_na, l_na, o_ws, l_ws)
        if i == len(seq) - 1:
            # the smaller, second call also against the oracle
            O_ref, L_ref = oracle.attention(q.float(), k.float(), v.float(), w.softmax_scale(), causal)
            og = o_na.float().cpu().numpy()
            lg = l_na.cpu().numpy().astype(np.float64)
            assert float(np.max(np.abs(og - O_ref.reshape(og.shape)))) <= 1.5e-2
            L_ref = L_ref.reshape(lg.shape)
            fin = np.isfinite(L_ref)
            assert np.array_equal(np.isfinite(lg), fin)
            assert float(np.max(np.abs(lg[fin] - L_ref[fin]))) <= 1e-3


def test_noalloc_prefill_plan():
    # a plan that needs no partials runs the prefill, as attn_fwd does
    w, q, k, v = _inputs(2, 8, 8, 1100, 1500, False, 41)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    assert attn.attn_fwd_choose_plan(qg, kg, vg).method == attn.ATTN_PLAN_PREFILL
    o_na, l_na = _noalloc(qg, kg, vg, w)
    o_ws, l_ws = attn.attn_fwd(qg, kg, vg, w.softmax_scale(), False)
    torch.cuda.synchronize()
    _close(o_na, l_na, o_ws, l_ws)


def test_noalloc_rejects_plan_beyond_array():
    # 511 query tiles of 128 rows (73 heads x 896 rows) and long rows: a split prefill
    # of two chunks whose partials (65408 rows x 2 chunks x 520 bytes) exceed 64 MiB
    w, q, k, v = _inputs(1, 73, 1, 896, 16384, False, 42)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    plan = attn.attn_fwd_choose_plan(qg, kg, vg)
    if attn.attn_device_cu_count(0) != 256:
        pytest.skip("the shape is sized for a device of 256 compute units")
    assert plan.method == attn.ATTN_PLAN_PREFILL_SPLIT
    assert plan.workspace_bytes > attn.NOALLOC_SCRATCH_BYTES
    out = torch.full(tuple(qg.shape), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.attn_fwd_noalloc(qg, kg, vg, out=out)
    assert e.value.status == attn.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was enqueued
