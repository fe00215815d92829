"""The prefill kernel over key chunks (attn_fwd_prefill_splitk) followed by
attn_splitk_combine, and attn_fwd where the planner picks that path, against
the fp64 oracle (Neptune notes, section 6: per-chunk partial results merged by
their log-sum-exp; the forward itself is the Mirage lecture's online-softmax
attention).  Chunks are whole 64-key tiles, C = 64 * ceil(Lk / (64 * S)), so
the cases cover ragged last chunks, empty trailing chunks, rows that see no key
of a chunk (causal, window, Lq > Lk) and every bias kind."""
import numpy as np
import pytest
import torch

import oracle
import synth
import online_softmax_fusion_amd as attn

from test_parity_gpu import compare, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


CASES = [
    # B, Hq, Hkv, Lq, Lk, D, causal, bias, softcap, window, S
    (1, 2, 2, 300, 1000, 128, True, "none", 0.0, None, 3),
    (2, 4, 2, 130, 700, 64, False, "alibi", 0.0, None, 4),
    (1, 2, 1, 200, 5000, 128, True, "dense_f32", 0.0, None, 5),
    (1, 2, 2, 129, 900, 64, False, "dense_bf16", 0.0, None, 2),
    (1, 2, 2, 256, 900, 128, True, "none", 5.0, None, 2),
    (1, 2, 2, 230, 2000, 128, True, "none", 0.0, (300, 0), 6),
    (1, 1, 1, 64, 100, 128, False, "none", 0.0, None, 8),      # chunks 2..7 empty
    (1, 2, 2, 300, 150, 128, True, "none", 0.0, None, 2),      # Lq > Lk: rows without keys
    (1, 4, 4, 1, 4100, 128, False, "none", 0.0, None, 16),     # one query row
    (1, 4, 2, 200, 1500, 128, True, "alibi", 0.0, None, 3),    # causal ALiBi, folded form
    (1, 2, 2, 140, 900, 128, True, "none", 50.0, None, 3),     # cap by the exp form
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_prefill_splitk_parity(case):
    B, Hq, Hkv, Lq, Lk, D, causal, bias, cap, window, S = case
    print("split prefill case", case, flush=True)
    w, q, k, v, gkw, okw = inputs(B, Hq, Hkv, Lq, Lk, D, "bf16", causal, bias, seed=41 + S)
    mods = {"softcap": cap, "window": window}
    op, mp, lp = attn.attn_fwd_prefill_splitk(q.cuda(), k.cuda(), v.cuda(), S, w.softmax_scale(), causal,
                                              **gkw, **mods)
    o, lse = attn.attn_splitk_combine(op, mp, lp, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # a chunk a row cannot see leaves m = -inf, l = 0, o = 0
    m, l = mp.cpu(), lp.cpu()
    assert torch.all((m == -float("inf")) == (l == 0)), "m = -inf exactly where l = 0"
    assert torch.all(op.cpu()[l == 0] == 0)
    O_ref, L_ref = oracle.attention(q, k, v, w.softmax_scale(), causal, softcap=cap, window=window, **okw)
    compare(o, lse, O_ref, L_ref, "bf16", str(case))


def test_prefill_splitk_matches_prefill_up_to_rounding():
    # one chunk is the plain prefill with the normalisation moved to the combine
    w, q, k, v, _, _ = inputs(1, 4, 2, 260, 777, 128, "bf16", True, "none", seed=3)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = attn.attn_fwd_prefill(q, k, v, w.softmax_scale(), True)
    op, mp, lp = attn.attn_fwd_prefill_splitk(q, k, v, 1, w.softmax_scale(), True)
    o2, l2 = attn.attn_splitk_combine(op, mp, lp, out_dtype=torch.bfloat16)
    assert float((o1.float() - o2.float()).abs().max()) <= 2 ** -8
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l2))
    assert float((l1[fin] - l2[fin]).abs().max()) <= 1e-5


def test_attn_fwd_runs_split_prefill():
    # R = 8 * ceil(1100 / 32) = 280 row blocks (no grouped split-K); 8 * 9
    # query tiles of 128 rows leave CUs idle: the planner splits the keys
    B, Hq, Hkv, Lq, Lk = 1, 8, 8, 1100, 5000
    w, q, k, v, _, _ = inputs(B, Hq, Hkv, Lq, Lk, 128, "bf16", True, "none", seed=9)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    plan = attn.attn_fwd_choose_plan(q, k, v, w.softmax_scale(), True, cu_count=256)
    assert plan.method == attn.ATTN_PLAN_PREFILL_SPLIT and plan.num_splits >= 2
    o, lse = attn.attn_fwd(q, k, v, w.softmax_scale(), True)
    torch.cuda.synchronize()
    local = [0, 1, 127, 128, 500, 1023, 1024, 1099]
    rows = np.array([h * Lq + i for h in range(Hq) for i in local], dtype=np.int64)
    O_ref, L_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), w.softmax_scale(), True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    compare(o.reshape(-1, 128)[idx], lse.reshape(-1)[idx], O_ref, L_ref, "bf16", "attn_fwd split prefill")


def test_prefill_splitk_rejects_fp32():
    w, q, k, v, _, _ = inputs(1, 1, 1, 64, 128, 64, "f32", False, "none")
    with pytest.raises(attn.AttnError):
        attn.attn_fwd_prefill_splitk(q.cuda(), k.cuda(), v.cuda(), 2, w.softmax_scale(), False)


def test_attn_fwd_split_prefill_graph_replay():
    """attn_fwd on the split-prefill plan (prefill over key chunks + combine)
    captured in a HIP graph gives the eager result on every replay, with other
    eager work between replays."""
    w, q, k, v, _, _ = inputs(1, 8, 8, 1100, 5000, 128, "bf16", True, "none", seed=13)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    sc = w.softmax_scale()
    plan = attn.attn_fwd_choose_plan(q, k, v, sc, True)
    assert plan.method == attn.ATTN_PLAN_PREFILL_SPLIT
    ws = torch.empty((plan.workspace_bytes,), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((1, 8, 1100), dtype=torch.float32, device="cuda")

    def step():
        attn.attn_fwd(q, k, v, sc, True, out=o, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        o.zero_()
        lse.zero_()
        attn.attn_fwd(q * 0.5, k, v, sc, True)   # unrelated eager work on the same plan
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "replay %d" % r
