"""The algorithmic FLOP and byte counts used by bench.py, pinned to the numbers
printed in the CMU 15-779 Lecture 11 (Mirage) notes -- section 1.2 / section 10
(one head, N=4096, d=128, bf16) and section 12 exercise 6 (GQA decode traffic)
-- and to brute-force counts of the causal mask."""
import json
import os

import numpy as np
import pytest

import bench
import synth


@pytest.fixture(scope="module")
def numbers(golden_dir):
    with open(os.path.join(golden_dir, "roofline_numbers.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (5, 5), (7, 12), (12, 7), (1, 9), (9, 1), (64, 64), (0, 5), (5, 0)])
def test_visible_pairs_brute(Lq, Lk):
    pos = np.arange(Lq)[:, None] + (Lk - Lq)
    brute = int(np.sum(np.arange(Lk)[None, :] <= pos)) if Lq and Lk else 0
    assert bench.visible_pairs(Lq, Lk, True) == brute
    assert bench.visible_pairs(Lq, Lk, False) == Lq * Lk


@pytest.mark.parametrize("Lq,Lk,causal,window", [
    (9, 9, True, (3, -1)), (7, 12, False, (2, 4)), (12, 7, True, (0, 0)), (10, 10, False, (-1, 2)),
    (5, 20, True, (100, 100)), (64, 64, True, (15, -1)), (3, 40, False, (5, -1))])
def test_visible_pairs_window_brute(Lq, Lk, causal, window):
    pos = np.arange(Lq)[:, None] + (Lk - Lq)
    keys = np.arange(Lk)[None, :]
    vis = np.ones((Lq, Lk), bool)
    if causal:
        vis &= keys <= pos
    if window[0] >= 0:
        vis &= keys >= pos - window[0]
    if window[1] >= 0:
        vis &= keys <= pos + window[1]
    assert bench.visible_pairs(Lq, Lk, causal, window) == int(vis.sum())


def test_head_matmul_flops(numbers):
    h = numbers["head"]
    f = bench.attention_flops(1, 1, h["N"], h["N"], h["d"], False)
    assert abs(f / 1e9 - h["matmul_GFLOP"]) < 0.05


def test_head_traffic(numbers):
    h = numbers["head"]
    N, d, e = h["N"], h["d"], h["bytes_per_elem"]
    nxn = 2 * N * N * e                                  # write once, read once
    flash = bench.prefill_bytes(1, 1, 1, N, N, d, e, e) - N * 4   # Q, K, V in, O out (no LSE)
    assert round(nxn / 1e6) == h["nxn_write_plus_read_MB"]
    assert abs(flash / 1e6 - h["flash_total_MB"]) < 0.05
    assert round((nxn + flash) / 1e6) == h["graph_level_total_MB"]
    assert round((nxn + flash) / flash) == h["reduction_factor"]


def test_gqa_exercise(numbers):
    g = numbers["gqa"]
    kv = 2 * g["batch"] * g["kv_heads"] * g["context"] * g["d"] * g["bytes_per_elem"]
    assert round(kv / 1e6) == g["kv_MB"]
    per_q = kv * g["q_heads_per_group"]
    assert round(per_q / 1e6) == g["per_query_head_MB"]
    assert round(per_q / (g["bandwidth_TBps"] * 1e12) * 1e6) == g["per_query_head_us"]
    assert round(kv / (g["bandwidth_TBps"] * 1e12) * 1e6) == g["grouped_us"]
    # our decode byte count reads each K/V element once per group, like the grouped form
    Hq = g["kv_heads"] * g["q_heads_per_group"]
    step = bench.decode_partial_kernel_bytes(g["batch"], Hq, g["kv_heads"], 1, g["context"], g["d"], 1)
    assert step - kv == g["batch"] * Hq * g["d"] * 2 + g["batch"] * Hq * (g["d"] + 2) * 4


def test_workload_counts():
    w = synth.C2_CAUSAL
    assert bench.attention_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, True) == 549_890_031_616
    w = synth.C5_PREFILL
    assert round(bench.attention_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, True) / 1e9, 2) == 2199.09
    w = synth.C4_DECODE
    assert bench.decode_step_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, 32) == 2_164_787_200


def test_backward_flops_are_five_products():
    # five products of 2*d FLOP per visible pair: 2.5 times the forward's two
    for causal, window in ((False, None), (True, None), (True, (7, -1))):
        f = bench.attention_flops(2, 3, 40, 50, 64, causal, window)
        b = bench.backward_flops(2, 3, 40, 50, 64, causal, window)
        assert 2 * b == 5 * f
    assert bench.backward_flops(4, 32, 4096, 4096, 128, False) == 10 * 128 * 4 * 32 * 4096 * 4096


def test_l2norm_bytes():
    # x read once, y written once, a 4-byte norm per row
    assert bench.l2norm_bytes(32768, 4096, 2, 2) == 32768 * 4096 * 4 + 32768 * 4
    assert bench.l2norm_bytes(8, 4194304, 4, 4) == 8 * 4194304 * 8 + 32


def test_source_digest_ignores_comments_only():
    # the traffic table is keyed on the code the compiler sees: comment and
    # whitespace edits keep an entry, any change to the code drops it
    src = 'int a = 1; // one\n/* block\n comment */ const char *s = "// kept";\n'
    assert bench.code_text(src) == bench.code_text(src.replace("// one", "// other").replace("\n", "\n\n  "))
    assert bench.code_text(src) != bench.code_text(src.replace("a = 1", "a = 2"))
    assert "// kept" in bench.code_text(src)
    assert bench.code_text("x = '/'; /* c */ y") == "x = '/'; y"


def test_dense_bias_bytes():
    """Distinct bf16 bias elements of the visible pairs (the batch shares the
    [H, L, L] tensor): for the dense-bias ALiBi workload (B=2, H=16, L=8192,
    causal) that is 16*L(L+1)/2 elements, the ~1.07 GB of extra reads the
    scope table names; with Q, K, V, O and LSE the roofline time at 8 TB/s
    stays below the matrix work's at 2.5 PFLOP/s."""
    w = synth.C3_DENSE
    L = w.Lq
    assert bench.dense_bias_bytes(w) == w.Hq * (L * (L + 1) // 2) * 2
    assert abs(bench.dense_bias_bytes(w) - 1.07e9) / 1.07e9 < 0.01
    nbytes = bench.prefill_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D) + bench.dense_bias_bytes(w)
    flops = bench.attention_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, w.causal, w.window)
    assert nbytes / 8e12 < flops / 2.5e15


def test_stats_ms_percentiles():
    d = sorted(float(x) for x in range(1, 21))     # 1 .. 20
    s = bench._stats_ms(d)
    assert s == {"mean": 10.5, "p10": 3.0, "p50": 11.0, "p90": 19.0}


def test_alibi_bias_tensor_matches_slopes():
    """The dense form of the ALiBi workload holds -slope_h * |i + Lk - Lq - j|."""
    w = synth.C3_DENSE.with_(Hq=3, Lq=5, Lk=9)
    b = synth.alibi_bias_tensor(w, "f32")
    sl = synth.alibi_slopes(3).double()
    for h in range(3):
        for i in range(5):
            for j in range(9):
                want = -float(sl[h]) * abs(i + 4 - j)
                assert abs(float(b[h, i, j]) - want) <= 1e-6 * max(1.0, abs(want))
