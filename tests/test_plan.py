"""The automatic choice of parallel dimensions (attn_fwd_choose_plan), on the
CPU: the plan is a pure host function of the shapes.

MEASURED is the outcome of timing the three forward paths on one MI355X (256
compute units) over 108 shapes, each causal and non-causal (bench.py
--plan-sweep): for every (Lk, B, Hq, Hkv) and query length, the paths whose
time (at their best split count) was within 10% of the fastest path's in both
runs: P = prefill kernel, K = grouped split-K (decode kernel and combine),
S = prefill kernel over key chunks and combine.  The planner must pick one of
them in every case."""
import ctypes

import pytest

import online_softmax_fusion_amd as attn

OK, INVALID, UNSUPPORTED = attn.ATTN_OK, attn.ATTN_ERR_INVALID_ARG, attn.ATTN_ERR_UNSUPPORTED

MEASURED = [
    # Lk, B, Hq, Hkv, "Lq:paths ..."
    (4096, 1, 8, 8, "1:KS 4:KS 16:KS 64:KS 128:KS 256:KS 512:S 1024:S 2048:S"),
    (4096, 1, 32, 8, "1:KS 4:KS 16:KS 64:KS 128:S 256:S 512:S 1024:P 2048:P"),
    (4096, 1, 64, 8, "1:KS 4:KS 16:KS 64:KS 128:S 256:S 512:P 1024:P 2048:P"),
    (4096, 4, 8, 8, "1:KS 4:KS 16:KS 64:KS 128:S 256:S 512:S 1024:P 2048:P"),
    (4096, 4, 32, 8, "1:K 4:K 16:K 64:S 128:S 256:P 512:P 1024:P 2048:P"),
    (4096, 4, 64, 8, "1:K 4:K 16:K 64:PS 128:P 256:P 512:P 1024:P 2048:P"),
    (32768, 1, 8, 8, "1:KS 4:KS 16:KS 64:S 128:S 256:S 512:S 1024:S 2048:S"),
    (32768, 1, 32, 8, "1:K 4:K 16:K 64:S 128:S 256:S 512:S 1024:PS 2048:PS"),
    (32768, 1, 64, 8, "1:K 4:K 16:K 64:S 128:S 256:S 512:PS 1024:PS 2048:P"),
    (32768, 4, 8, 8, "1:KS 4:KS 16:KS 64:KS 128:S 256:S 512:S 1024:S 2048:P"),
    (32768, 4, 32, 8, "1:K 4:K 16:K 64:S 128:S 256:S 512:PS 1024:P 2048:P"),
    (32768, 4, 64, 8, "1:K 4:K 16:K 64:S 128:S 256:PS 512:P 1024:P 2048:P"),
]

METHOD = {attn.ATTN_PLAN_PREFILL: "P", attn.ATTN_PLAN_SPLITK: "K", attn.ATTN_PLAN_PREFILL_SPLIT: "S"}

P = 0x100000


@pytest.fixture(scope="module")
def lib():
    return attn.load_library()


def args(B, Hq, Hkv, Lq, Lk, D=128, dtype=attn.ATTN_BF16, causal=0):
    a = attn.AttnFwdArgs()
    a.B, a.Hq, a.Hkv, a.Lq, a.Lk, a.D = B, Hq, Hkv, Lq, Lk, D
    a.dtype, a.causal = dtype, causal
    a.q, a.k, a.v, a.o, a.lse = P, 2 * P, 3 * P, 4 * P, 5 * P
    a.q_strides = (ctypes.c_int64 * 3)(Hq * Lq * D, Lq * D, D)
    a.k_strides = (ctypes.c_int64 * 3)(Hkv * Lk * D, Lk * D, D)
    a.v_strides = (ctypes.c_int64 * 3)(Hkv * Lk * D, Lk * D, D)
    a.o_strides = (ctypes.c_int64 * 3)(Hq * Lq * D, Lq * D, D)
    a.o_dtype = dtype
    a.scale = 0.088
    return a


def plan_of(lib, a, cu=256):
    p = attn.AttnFwdPlan()
    st = lib.attn_fwd_choose_plan(ctypes.byref(a), cu, ctypes.byref(p))
    return st, p


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("row", MEASURED, ids=lambda r: "Lk%d-B%d-H%d/%d" % r[:4])
def test_plan_picks_a_measured_fast_path(lib, row, causal):
    Lk, B, Hq, Hkv, outcomes = row
    for item in outcomes.split():
        Lq, ok = item.split(":")
        st, p = plan_of(lib, args(B, Hq, Hkv, int(Lq), Lk, causal=causal))
        assert st == OK
        assert METHOD[p.method] in ok, (row[:4], Lq, METHOD[p.method], ok)


def test_split_plan_details(lib):
    # B1 H8 Lq 16 Lk 32768: 8 row blocks, the split chooser fills 256 CUs with 32 chunks
    st, p = plan_of(lib, args(1, 8, 8, 16, 32768))
    assert st == OK and p.method == attn.ATTN_PLAN_SPLITK
    assert p.num_splits == lib.attn_decode_choose_splits(1, 8, 8, 16, 32768, 256) == 32
    assert p.workspace_bytes == lib.attn_decode_partial_bytes(1, 8, 16, 128, 32)
    # B1 H8 Lq 2048 Lk 32768: 128 query tiles, 4 key chunks give two workgroups per CU
    st, p = plan_of(lib, args(1, 8, 8, 2048, 32768))
    assert st == OK and p.method == attn.ATTN_PLAN_PREFILL_SPLIT
    assert p.num_splits == lib.attn_prefill_choose_splits(1, 8, 2048, 32768, 256) == 4
    assert p.workspace_bytes == lib.attn_decode_partial_bytes(1, 8, 2048, 128, 4)
    # chunks keep at least 1024 keys: B1 H8 Lq 128 Lk 4096 gets 4, not 64
    assert lib.attn_prefill_choose_splits(1, 8, 128, 4096, 256) == 4
    # a grid with a workgroup per CU splits only into chunks of 8192 keys or more
    assert lib.attn_prefill_choose_splits(1, 32, 1024, 4096, 256) == 1
    assert lib.attn_prefill_choose_splits(1, 32, 1024, 32768, 256) == 2
    # prefill plans need no workspace
    st, p = plan_of(lib, args(4, 32, 32, 4096, 4096))
    assert st == OK and p.method == attn.ATTN_PLAN_PREFILL and p.num_splits == 0 and p.workspace_bytes == 0


def test_plan_boundary_follows_cu_count(lib):
    # decode-like: R = B * Hkv * ceil(G * Lq / 32) = 8 row blocks
    a = args(1, 8, 8, 16, 4096)
    assert plan_of(lib, a, 256)[1].method == attn.ATTN_PLAN_SPLITK
    assert plan_of(lib, a, 8)[1].method == attn.ATTN_PLAN_SPLITK
    assert plan_of(lib, a, 7)[1].method == attn.ATTN_PLAN_PREFILL
    assert plan_of(lib, a, 0)[1].method == attn.ATTN_PLAN_SPLITK     # 0: the MI355X's 256
    # 128 query tiles of 128 rows: split while they leave CUs idle
    a = args(1, 8, 8, 2048, 4096)
    assert plan_of(lib, a, 256)[1].method == attn.ATTN_PLAN_PREFILL_SPLIT
    assert plan_of(lib, a, 129)[1].method == attn.ATTN_PLAN_PREFILL_SPLIT
    assert plan_of(lib, a, 128)[1].method == attn.ATTN_PLAN_PREFILL


def test_plan_fp32_and_empty_keys_use_prefill(lib):
    assert plan_of(lib, args(1, 8, 8, 16, 4096, dtype=attn.ATTN_F32))[1].method == attn.ATTN_PLAN_PREFILL
    assert plan_of(lib, args(1, 8, 8, 16, 0))[1].method == attn.ATTN_PLAN_PREFILL


def test_plan_validates(lib):
    a = args(1, 8, 8, 16, 4096)
    a.Hq = 7
    assert plan_of(lib, a)[0] == INVALID
    a = args(1, 8, 8, 16, 4096, D=96)
    assert plan_of(lib, a)[0] == UNSUPPORTED
    assert lib.attn_fwd_choose_plan(ctypes.byref(args(1, 8, 8, 16, 4096)), 256, None) == INVALID
    a = args(1, 8, 8, 16, 4096)
    a.o = None
    assert lib.attn_fwd(ctypes.byref(a), None, 0, None) == INVALID


def test_prefill_split_count_contract(lib):
    # include/attn.h: enough (query tile, chunk) workgroups for two per CU, at
    # least 1024 keys per chunk, and on a grid with a workgroup per CU only
    # chunks of 8192 keys or more; 1 means no split
    for cu in (0, 80, 256):
        c = cu if cu > 0 else 256
        for B, Hq in ((1, 1), (1, 8), (2, 16), (4, 64)):
            for Lq in (1, 100, 128, 1000, 4096):
                for Lk in (1, 1023, 2048, 5000, 32768, 100000):
                    S = lib.attn_prefill_choose_splits(B, Hq, Lq, Lk, cu)
                    blocks = B * Hq * -(-Lq // 128)
                    assert S >= 1
                    if S == 1:
                        continue
                    chunk = attn.prefill_chunk_length(Lk, S)
                    assert Lk // S >= 1024
                    assert blocks * (S - 1) < 2 * c   # no more chunks than two workgroups per CU need
                    assert blocks < c or chunk >= 8192
    assert lib.attn_prefill_choose_splits(0, 8, 128, 4096, 256) == 1
