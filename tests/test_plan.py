"""The automatic choice of parallel dimensions (attn_fwd_choose_plan), on the
CPU: the plan is a pure host function of the shapes.

MEASURED is the outcome of timing both paths on one MI355X (256 compute
units) over 108 shapes, each causal and non-causal (216 runs, identical
outcome for both): for every (Lk, B, Hq, Hkv) the query lengths at which the
grouped split-K path (best split count) beat the prefill kernel, and those at
which it lost.  The planner must pick the faster path in every case."""
import ctypes

import pytest

import online_softmax_fusion_amd as attn

OK, INVALID, UNSUPPORTED = attn.ATTN_OK, attn.ATTN_ERR_INVALID_ARG, attn.ATTN_ERR_UNSUPPORTED

MEASURED = [
    # Lk, B, Hq, Hkv, Lq where split-K was faster, Lq where prefill was faster
    (4096, 1, 8, 8, (1, 4, 16, 64, 128, 256, 512, 1024), (2048,)),
    (4096, 1, 32, 8, (1, 4, 16, 64, 128, 256), (512, 1024, 2048)),
    (4096, 1, 64, 8, (1, 4, 16, 64, 128), (256, 512, 1024, 2048)),
    (4096, 4, 8, 8, (1, 4, 16, 64, 128, 256), (512, 1024, 2048)),
    (4096, 4, 32, 8, (1, 4, 16, 64), (128, 256, 512, 1024, 2048)),
    (4096, 4, 64, 8, (1, 4, 16), (64, 128, 256, 512, 1024, 2048)),
    (32768, 1, 8, 8, (1, 4, 16, 64, 128, 256, 512, 1024), (2048,)),
    (32768, 1, 32, 8, (1, 4, 16, 64, 128, 256), (512, 1024, 2048)),
    (32768, 1, 64, 8, (1, 4, 16, 64, 128), (256, 512, 1024, 2048)),
    (32768, 4, 8, 8, (1, 4, 16, 64, 128, 256), (512, 1024, 2048)),
    (32768, 4, 32, 8, (1, 4, 16, 64), (128, 256, 512, 1024, 2048)),
    (32768, 4, 64, 8, (1, 4, 16), (64, 128, 256, 512, 1024, 2048)),
]

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
def test_plan_picks_the_measured_faster_path(lib, row, causal):
    Lk, B, Hq, Hkv, splitk_lqs, prefill_lqs = row
    for Lq, want in [(l, attn.ATTN_PLAN_SPLITK) for l in splitk_lqs] + [(l, attn.ATTN_PLAN_PREFILL) for l in prefill_lqs]:
        st, p = plan_of(lib, args(B, Hq, Hkv, Lq, Lk, causal=causal))
        assert st == OK
        assert p.method == want, (row, Lq)


def test_split_plan_details(lib):
    # B1 H8 Lq 16 Lk 32768: 8 row blocks, the split chooser fills 256 CUs with 32 chunks
    st, p = plan_of(lib, args(1, 8, 8, 16, 32768))
    assert st == OK and p.method == attn.ATTN_PLAN_SPLITK
    assert p.num_splits == lib.attn_decode_choose_splits(1, 8, 8, 16, 32768, 256) == 32
    assert p.workspace_bytes == lib.attn_decode_partial_bytes(1, 8, 16, 128, 32)
    # prefill plans need no workspace
    st, p = plan_of(lib, args(4, 32, 32, 4096, 4096))
    assert st == OK and p.method == attn.ATTN_PLAN_PREFILL and p.num_splits == 0 and p.workspace_bytes == 0


def test_plan_boundary_follows_cu_count(lib):
    # R = B * Hkv * ceil(G * Lq / 32): 1 * 8 * 16 = 128 row blocks
    a = args(1, 8, 8, 512, 4096)
    assert plan_of(lib, a, 256)[1].method == attn.ATTN_PLAN_SPLITK
    assert plan_of(lib, a, 128)[1].method == attn.ATTN_PLAN_SPLITK
    assert plan_of(lib, a, 127)[1].method == attn.ATTN_PLAN_PREFILL
    assert plan_of(lib, a, 0)[1].method == attn.ATTN_PLAN_SPLITK     # 0: the MI355X's 256


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
