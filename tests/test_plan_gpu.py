"""attn_fwd (the planned forward) against the fp64 oracle on shapes where the
plan is split-K and where it is prefill (GPU).  Tolerances as for the other
bf16 forward tests: 1.5e-2 on O, 1e-3 on LSE."""
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


CASES = [
    # B, Hq, Hkv, Lq, Lk, causal, bias, softcap, window, expected plan
    (1, 8, 8, 16, 4096, False, "none", 0.0, None, attn.ATTN_PLAN_SPLITK),
    (1, 32, 8, 100, 3000, True, "none", 0.0, None, attn.ATTN_PLAN_PREFILL_SPLIT),  # Lq < Lk, end-aligned
    (2, 4, 4, 700, 700, True, "alibi", 0.0, None, attn.ATTN_PLAN_SPLITK),     # 176 row blocks, 2 chunks
    (1, 8, 2, 33, 5000, False, "none", 20.0, (300, 40), attn.ATTN_PLAN_PREFILL_SPLIT),
    (1, 16, 4, 64, 2048, True, "dense_f32", 0.0, (511, -1), attn.ATTN_PLAN_PREFILL_SPLIT),
    (4, 16, 16, 300, 300, True, "none", 0.0, None, attn.ATTN_PLAN_PREFILL),
    (2, 8, 8, 1100, 1500, False, "alibi", 0.0, None, attn.ATTN_PLAN_PREFILL),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_attn_fwd_parity(case):
    B, Hq, Hkv, Lq, Lk, causal, bias, softcap, window, want = case
    print("attn_fwd case", case, flush=True)
    w = synth.Workload("plan", B, Hq, Hkv, Lq, Lk, 128, "bf16", causal, bias, 17, softcap=softcap, window=window)
    q, k, v = synth.make_qkv(w)
    gkw, okw = {}, {}
    if bias == "alibi":
        sl = synth.alibi_slopes(Hq)
        gkw["alibi_slopes"], okw["alibi_slopes"] = sl.cuda(), sl
    elif bias == "dense_f32":
        bt = synth.make_dense_bias(w, (Hq, Lq, Lk), "f32")
        gkw["bias"], okw["bias"] = bt.cuda(), bt
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    plan = attn.attn_fwd_choose_plan(qg, kg, vg, w.softmax_scale(), causal, softcap=softcap, window=window, **gkw)
    assert plan.method == want
    o, lse = attn.attn_fwd(qg, kg, vg, w.softmax_scale(), causal, softcap=softcap, window=window, **gkw)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q.float(), k.float(), v.float(), w.softmax_scale(), causal, softcap=softcap,
                                    window=window, **okw)
    O_ref = O_ref.reshape(B, Hq, Lq, 128)
    L_ref = L_ref.reshape(B, Hq, Lq)
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(og - O_ref))) <= 1.5e-2
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(lg), fin)
    if fin.any():
        assert float(np.max(np.abs(lg[fin] - L_ref[fin]))) <= 1e-3


def test_attn_fwd_rejects_small_workspace():
    w = synth.Workload("plan", 1, 8, 8, 16, 4096, 128, "bf16", False, "none", 18)
    q, k, v = (t.cuda() for t in synth.make_qkv(w))
    plan = attn.attn_fwd_choose_plan(q, k, v)
    assert plan.method == attn.ATTN_PLAN_SPLITK and plan.workspace_bytes > 0
    small = torch.empty((plan.workspace_bytes - 16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.attn_fwd(q, k, v, workspace=small)
    assert e.value.status == attn.ATTN_ERR_WORKSPACE
    exact = torch.empty((plan.workspace_bytes,), dtype=torch.uint8, device="cuda")
    o1, l1 = attn.attn_fwd(q, k, v, workspace=exact)
    o2, l2 = attn.attn_fwd_prefill(q, k, v)
    torch.cuda.synchronize()
    assert float((o1.float() - o2.float()).abs().max()) <= 1.5e-2
    assert float((l1 - l2).abs().max()) <= 1e-3
