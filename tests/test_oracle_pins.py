"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself:

* the 2x4 max / exp / sum worked example of "Neptune论文浅读" section 3, with
  closed-form values (tests/golden/softmax_2x4.json), run through the three
  printed program shapes (three loops, naive fusion, repaired fusion) and
  through the oracle with scores set to the example row;
* the online softmax of the CANN FlashAttention post (section on the online
  softmax), in its corrected reading, against the two-pass form;
* invariants fixed by the stable-softmax definition (Neptune notes section 2):
  rows of the softmax sum to 1, constant V gives constant O, a constant bias
  shifts LSE and leaves O alone, Q = 0 gives the mean of the visible values with
  LSE = ln(count), causal row 0 returns v_0;
* an exact case: two keys with bias (0, ln 3) give weights (1/4, 3/4);
* brute force: the full score matrix through scipy's softmax and logsumexp
  (a library routine) at N <= 64, covering scale, causal alignment with
  Lq != Lk, GQA, ALiBi and dense bias;
* large logits stay finite (Mirage lecture section 5.5: q and K scaled by 40);
* the split-K combine against the unsplit oracle over several chunkings, with
  arbitrary per-chunk reference values ("subtracting any m gives the same",
  Mirage lecture section 5.5) and empty chunks;
* the backward (dQ, dK, dV) against central finite differences of the scipy
  brute force, and invariants: value gradients add up to the output gradients,
  key gradients add up to zero, equal keys give dQ = 0, Q = 0 gives dV in
  closed form;
* the row L2 norm: closed forms (3-4-5 at scales 2^100 and 2^-120, ones),
  exact power-of-two scale invariance, unit rows, zero rows, a strided input,
  numpy.linalg.norm on random rows;
* planted mistakes: copies of the oracle with a plausible error each (wrong kv
  head, dropped scale, bias sign, causal off-by-one, log base, combine weight,
  dropped Delta, missing cap slope, wrong head group in the backward, ...)
  are compiled and must fail these pins.
"""
import json
import functools
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle

RNG = np.random.default_rng(20261202)


# ----------------------------------------------------------------------------
# independent brute force: full score matrix through scipy
# ----------------------------------------------------------------------------
def brute(q, k, v, scale, causal=False, bias=None, slopes=None, softcap=0.0, window=None):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=1)
    vv = np.repeat(v, G, axis=1)
    S = scale * np.matmul(q, np.swapaxes(kk, -1, -2))
    if softcap > 0:
        S = softcap * np.tanh(S / softcap)
    pos = np.arange(Lq)[:, None] + (Lk - Lq)
    keys = np.arange(Lk)[None, :]
    if bias is not None:
        S = S + np.asarray(bias, dtype=np.float64)
    if slopes is not None:
        S = S - np.asarray(slopes, dtype=np.float64)[None, :, None, None] * np.abs(pos - keys)
    if causal:
        S = np.where(keys > pos, -np.inf, S)
    if window is not None:
        wl, wr = window
        if wl >= 0:
            S = np.where(keys < pos - wl, -np.inf, S)
        if wr >= 0:
            S = np.where(keys > pos + wr, -np.inf, S)
    lse = logsumexp(S, axis=-1)
    empty = np.isneginf(lse)
    S_safe = np.where(empty[..., None], 0.0, S)
    P = softmax(S_safe, axis=-1)
    P = np.where(empty[..., None], 0.0, P)
    O = np.matmul(P, vv)
    return O, lse


def rnd(*shape, scale=1.0):
    return (RNG.standard_normal(shape) * scale).astype(np.float32)


def assert_close(a, b, tol, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), what + ": infinity pattern differs"
    assert np.array_equal(a[~fin], b[~fin]), what + ": infinite values differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


# ----------------------------------------------------------------------------
# Neptune notes section 3: the 2x4 example; what each program shape computes,
# stated over whole rows (numpy), and the repair of section 4 as a merge
# ----------------------------------------------------------------------------
def three_loop(inp):
    """Three separate passes: the row max, then sum_j exp(x_j - max)."""
    x = np.asarray(inp, dtype=np.float64)
    m = x.max(axis=1)
    return m.tolist(), np.exp(x - m[:, None]).sum(axis=1).tolist()


def naive_fused(inp):
    """Exponentials taken inside the max pass without repair: term j is
    exp(x_j - max(x_0 .. x_j)), against the max seen so far, not the row's."""
    x = np.asarray(inp, dtype=np.float64)
    running = np.maximum.accumulate(x, axis=1)
    return x.max(axis=1).tolist(), np.exp(x - running).sum(axis=1).tolist()


def merge(a, b):
    """(m, s) states of two parts of a row combined with the repair function
    h(t, r, r') = t exp(r - r') of section 4: both sums are moved to the
    larger reference before they are added."""
    (m1, s1), (m2, s2) = a, b
    M = max(m1, m2)
    if M == -math.inf:
        return M, 0.0
    return M, s1 * math.exp(m1 - M) + s2 * math.exp(m2 - M)


def repaired_fused(inp, order="left"):
    """The fused single pass: every element is the state (x_j, 1), and the
    states are merged left to right ("left") or pairwise as a tree ("tree")."""
    out_m, out_s = [], []
    for row in inp:
        states = [(float(v), 1.0) for v in row]
        if order == "left":
            st = functools.reduce(merge, states, (-math.inf, 0.0))
        else:
            while len(states) > 1:
                states = [merge(states[i], states[i + 1]) if i + 1 < len(states) else states[i]
                          for i in range(0, len(states), 2)]
            st = states[0]
        out_m.append(st[0])
        out_s.append(st[1])
    return out_m, out_s


@pytest.fixture(scope="module")
def ex2x4(golden_dir):
    with open(os.path.join(golden_dir, "softmax_2x4.json")) as f:
        return json.load(f)


def test_golden_2x4_closed_form_digits(ex2x4):
    closed = (1 - math.exp(-4)) / (1 - math.exp(-1))
    for s in ex2x4["xsum"]:
        assert abs(s - closed) <= 1e-15
    assert abs(ex2x4["lse"][0] - (3 + math.log(closed))) <= 1e-15


def test_2x4_three_loop_matches_closed_form(ex2x4):
    xmax, xsum = three_loop(ex2x4["inp"])
    assert xmax == ex2x4["xmax"]
    for a, b in zip(xsum, ex2x4["xsum"]):
        assert abs(a - b) <= 1e-15


def test_2x4_naive_fusion_is_wrong_when_max_grows(ex2x4):
    _, xsum = naive_fused(ex2x4["inp"])
    assert xsum[0] == ex2x4["naive_fused_xsum"][0] == 4.0
    assert abs(xsum[0] - ex2x4["xsum"][0]) > 2.0
    assert abs(xsum[1] - ex2x4["naive_fused_xsum"][1]) <= 1e-15


def test_2x4_repaired_fusion_equals_three_loop(ex2x4):
    xmax, xsum = repaired_fused(ex2x4["inp"])
    assert xmax == ex2x4["xmax"]
    for a, b in zip(xsum, ex2x4["xsum"]):
        assert abs(a - b) <= 1e-15 * b


def test_2x4_repaired_fusion_random_rows():
    inp = RNG.standard_normal((2, 4)).tolist()
    _, s3 = three_loop(inp)
    for order in ("left", "tree"):
        _, sr = repaired_fused(inp, order)
        for a, b in zip(sr, s3):
            assert abs(a - b) <= 1e-15 * b


def test_oracle_reproduces_2x4_example(ex2x4):
    """Scores equal to the example rows: q = e_0, k_j = x_j e_0, scale 1, V = I."""
    inp = np.asarray(ex2x4["inp"], dtype=np.float32)
    for r in range(2):
        q = np.eye(4, dtype=np.float32)[0].reshape(1, 1, 1, 4)
        k = np.zeros((1, 1, 4, 4), np.float32)
        k[0, 0, :, 0] = inp[r]
        v = np.eye(4, dtype=np.float32).reshape(1, 1, 4, 4)
        O, lse = oracle.attention(q, k, v, 1.0)
        expect_p = np.exp(inp[r].astype(np.float64) - ex2x4["xmax"][r]) / ex2x4["xsum"][r]
        assert_close(O.reshape(4), expect_p, 1e-15, "softmax row")
        assert abs(lse.item() - ex2x4["lse"][r]) <= 1e-14


# ----------------------------------------------------------------------------
# CANN FA post: online softmax (corrected reading) == two-pass softmax_standard
# ----------------------------------------------------------------------------
def softmax_standard_weighted(x, vals):
    m = max(x)
    e = [math.exp(xi - m) for xi in x]
    tot = sum(e)
    return sum(ei * vi for ei, vi in zip(e, vals)) / tot


def softmax_online_weighted(x, vals):
    """running (m, l, o): both l and o are rescaled by exp(m - m_new); O = o / l."""
    m, l, o = -math.inf, 0.0, 0.0
    for xi, vi in zip(x, vals):
        m_new = max(m, xi)
        c = math.exp(m - m_new)
        l = l * c + math.exp(xi - m_new)
        o = o * c + math.exp(xi - m_new) * vi
        m = m_new
    return o / l


@pytest.mark.parametrize("n", [1, 2, 7, 64])
def test_online_equals_two_pass(n):
    for _ in range(20):
        x = (RNG.standard_normal(n) * 4).tolist()
        vals = RNG.standard_normal(n).tolist()
        a = softmax_online_weighted(x, vals)
        b = softmax_standard_weighted(x, vals)
        assert abs(a - b) <= 1e-13 * max(1.0, abs(b))


def test_printed_online_listing_is_garbled():
    """The CANN FlashAttention post's online-softmax listing (its online
    softmax section) multiplies o by the already-updated l and returns o
    without dividing by l.  Followed by hand on the scores x = (0, 1, 2) with
    values (1, 2, 3) -- the max grows at every step, so every repair factor is
    e^-1 -- it gives l = 1 + e^-1 + e^-2 and
        o = 3 + e^-1 (2 + e^-1 + e^-2)(1 + e^-1 + e^-2) = 4.38428...,
    while the softmax-weighted value is (1 + 2e + 3e^2) / (1 + e + e^2) =
    2.5752...; the corrected recurrence (reading 10) gives the latter."""
    e1, e2 = math.exp(-1.0), math.exp(-2.0)
    printed = 3.0 + e1 * (2.0 + e1 + e2) * (1.0 + e1 + e2)
    x, vals = [0.0, 1.0, 2.0], [1.0, 2.0, 3.0]
    good = softmax_standard_weighted(x, vals)
    assert abs(good - (1 + 2 * math.e + 3 * math.e ** 2) / (1 + math.e + math.e ** 2)) <= 1e-14
    assert abs(printed - 4.3842822) <= 1e-6 and abs(printed - good) > 1.0
    assert abs(softmax_online_weighted(x, vals) - good) <= 1e-14


# ----------------------------------------------------------------------------
# invariants of the definition
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    L = 24
    q, k = rnd(2, 3, L, L), rnd(2, 3, L, L)
    v = np.broadcast_to(np.eye(L, dtype=np.float32), (2, 3, L, L)).copy()
    O, _ = oracle.attention(q, k, v, 0.37, causal)
    assert np.all(O >= 0.0)
    assert np.max(np.abs(O.sum(-1) - 1.0)) <= 1e-14
    if causal:
        upper = np.triu(np.ones((L, L), bool), 1)
        assert np.all(O[..., upper] == 0.0)


def test_constant_v_gives_constant_o():
    q, k = rnd(1, 4, 33, 8, scale=3), rnd(1, 2, 40, 8, scale=3)
    v = np.full((1, 2, 40, 8), -1.75, np.float32)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625], np.float32)
    for kw in ({}, {"alibi_slopes": slopes}, {"bias": rnd(4, 33, 40)}):
        for causal in (False, True):
            O, lse = oracle.attention(q, k, v, 0.5, causal, **kw)
            assert np.max(np.abs(O + 1.75)) <= 1e-14
            assert np.all(np.isfinite(lse))


def test_constant_bias_shifts_lse_only():
    q, k, v = rnd(2, 2, 9, 8), rnd(2, 2, 13, 8), rnd(2, 2, 13, 8)
    O0, l0 = oracle.attention(q, k, v, 0.4, True)
    O1, l1 = oracle.attention(q, k, v, 0.4, True, bias=np.full((1,), 2.5, np.float32))
    assert_close(O1, O0, 1e-14, "O")
    assert_close(l1, l0 + 2.5, 1e-13, "LSE")


def test_two_keys_exact_weights():
    """q = 0 so every score is its bias; bias (0, ln 3) gives weights (1/4, 3/4)."""
    q = np.zeros((1, 1, 1, 4), np.float32)
    k = rnd(1, 1, 2, 4)
    v = np.array([[1, 0, 2, 0], [0, 1, 2, 4]], np.float32).reshape(1, 1, 2, 4)
    bias = np.array([0.0, math.log(3.0)], np.float32).reshape(1, 1, 1, 2)
    O, lse = oracle.attention(q, k, v, 1.0, bias=bias)
    b1 = float(np.float32(math.log(3.0)))
    w1 = math.exp(b1) / (1 + math.exp(b1))
    v64 = v.astype(np.float64)
    expect = (1 - w1) * v64[0, 0, 0] + w1 * v64[0, 0, 1]
    assert_close(O.reshape(4), expect, 1e-15, "O")
    assert abs(lse.item() - math.log(1 + math.exp(b1))) <= 1e-15
    assert abs(w1 - 0.75) < 1e-7


@pytest.mark.parametrize("Lq,Lk", [(16, 16), (5, 12), (1, 30)])
def test_zero_q_gives_mean_of_visible(Lq, Lk):
    q = np.zeros((1, 2, Lq, 8), np.float32)
    k, v = rnd(1, 2, Lk, 8), rnd(1, 2, Lk, 8)
    O, lse = oracle.attention(q, k, v, 0.9, True)
    for i in range(Lq):
        n = i + (Lk - Lq) + 1
        assert_close(O[0, :, i], v[0, :, :n].astype(np.float64).mean(1), 1e-14, "mean")
        assert np.max(np.abs(lse[0, :, i] - math.log(n))) <= 1e-14


def test_causal_row0_is_v0():
    q, k, v = rnd(2, 3, 10, 16), rnd(2, 3, 10, 16), rnd(2, 3, 10, 16)
    O, lse = oracle.attention(q, k, v, 0.25, True)
    assert_close(O[:, :, 0], v[:, :, 0].astype(np.float64), 1e-15, "O_0")
    s00 = 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64), k[:, :, 0].astype(np.float64))
    assert_close(lse[:, :, 0], s00, 1e-14, "LSE_0")


def test_decode_query_sees_all_keys():
    q, k, v = rnd(3, 4, 1, 16), rnd(3, 2, 50, 16), rnd(3, 2, 50, 16)
    a = oracle.attention(q, k, v, 0.25, True)
    b = oracle.attention(q, k, v, 0.25, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fully_masked_rows():
    """Lq > Lk with causal alignment to the end: the first Lq - Lk rows see nothing."""
    q, k, v = rnd(1, 2, 8, 4), rnd(1, 2, 5, 4), rnd(1, 2, 5, 4)
    O, lse = oracle.attention(q, k, v, 1.0, True)
    assert np.all(O[:, :, :3] == 0.0)
    assert np.all(np.isneginf(lse[:, :, :3]))
    assert np.all(np.isfinite(lse[:, :, 3:]))
    Ob, lb = brute(q, k, v, 1.0, True)
    assert_close(O, Ob, 1e-14, "O")
    assert_close(lse, lb, 1e-13, "LSE")


def test_empty_key_set():
    q = rnd(1, 1, 3, 4)
    k = np.zeros((1, 1, 0, 4), np.float32)
    O, lse = oracle.attention(q, k, k, 1.0)
    assert np.all(O == 0.0) and np.all(np.isneginf(lse))


# ----------------------------------------------------------------------------
# brute force through scipy
# ----------------------------------------------------------------------------
BRUTE_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, scale, causal, bias
    (1, 1, 1, 16, 16, 8, 0.35, False, None),
    (2, 2, 2, 17, 17, 16, 0.25, True, None),
    (1, 4, 2, 9, 31, 8, 0.5, True, None),
    (2, 8, 2, 1, 64, 16, 0.125, False, None),
    (1, 6, 3, 33, 20, 4, 1.0, True, "dense"),
    (2, 4, 4, 20, 45, 8, 0.3, True, "alibi"),
    (1, 4, 1, 64, 64, 64, 0.125, False, "alibi"),
    (2, 2, 1, 12, 12, 1, 2.0, False, "dense_b"),
]


# SoftCap and Window (Neptune notes section 9 names both operators; readings:
# cap = c * tanh(score / c) on the scaled score before any bias; window keeps
# keys p - left <= j <= p + right, negative = unbounded)
MOD_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, scale, causal, bias, softcap, window
    (1, 2, 1, 20, 20, 8, 1.5, False, None, 3.0, None),
    (2, 2, 2, 17, 30, 8, 2.0, True, "dense", 2.5, None),
    (1, 4, 2, 24, 24, 8, 0.5, True, None, 0.0, (5, -1)),
    (1, 2, 2, 19, 33, 4, 0.7, False, None, 0.0, (3, 6)),
    (2, 4, 4, 16, 40, 8, 0.4, True, "alibi", 4.0, (7, 0)),
    (1, 2, 1, 12, 12, 8, 0.9, False, None, 1.0, (0, 0)),
    (1, 1, 1, 10, 25, 4, 1.0, True, None, 0.0, (2, -1)),     # rows whose window is inside the causal range
    (1, 1, 1, 8, 8, 4, 1.0, False, None, 0.0, (-1, 2)),      # right bound only
]


def _mod_inputs(case, rng):
    B, Hq, Hkv, Lq, Lk, D, scale, causal, bias_kind, softcap, window = case
    q = (rng.standard_normal((B, Hq, Lq, D)) * 2).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, Lk, D)) * 2).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Lk, D)).astype(np.float32)
    kw, bkw = {"softcap": softcap, "window": window}, {"softcap": softcap, "window": window}
    if bias_kind == "dense":
        bias = rng.standard_normal((B, Hq, Lq, Lk)).astype(np.float32)
        kw["bias"] = bkw["bias"] = bias
    elif bias_kind == "alibi":
        slopes = np.power(2.0, -8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        kw["alibi_slopes"] = bkw["slopes"] = slopes
    return q, k, v, scale, causal, kw, bkw


@pytest.mark.parametrize("case", MOD_CASES, ids=[str(i) for i in range(len(MOD_CASES))])
def test_brute_force_softcap_window(case):
    q, k, v, scale, causal, kw, bkw = _mod_inputs(case, np.random.default_rng(23))
    O, lse = oracle.attention(q, k, v, scale, causal, **kw)
    Ob, lb = brute(q, k, v, scale, causal, **bkw)
    assert_close(O, Ob, 1e-12, "O")
    assert_close(lse, lb, 1e-12, "LSE")


def test_softcap_closed_form_two_keys():
    """tanh(ln(3) / 2) = (3 - 1) / (3 + 1) = 1/2, so with cap c = 2 a scaled
    score of ln 3 is capped to exactly 1: against a score of 0 the weights are
    e / (e + 1) and 1 / (e + 1), and LSE = ln(e + 1).  (ln 3 is stored in fp32,
    which moves the capped score by ~1e-7.)"""
    q = np.array([[[[1.0, 0.0]]]], np.float32)
    k = np.array([[[[np.log(3.0), 0.0], [0.0, 0.0]]]], np.float32)
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], np.float32)
    O, lse = oracle.attention(q, k, v, 1.0, softcap=2.0)
    e = np.e
    assert_close(O.reshape(2), np.array([e / (e + 1), 1 / (e + 1)]), 1e-7, "O")
    assert_close(lse.reshape(1), np.array([np.log(e + 1)]), 1e-7, "LSE")
    # a huge score saturates at the cap: weights e^c / (e^c + 1) for c = 1
    k2 = np.array([[[[1000.0, 0.0], [0.0, 0.0]]]], np.float32)
    O2, _ = oracle.attention(q, k2, v, 1.0, softcap=1.0)
    assert_close(O2.reshape(2), np.array([e / (e + 1), 1 / (e + 1)]), 1e-15, "saturated O")


def test_softcap_limit_and_bound():
    """A cap far above every score changes nothing (to fp64 rounding); with a
    cap c every weight ratio inside a row is at most e^(2c)."""
    rng = np.random.default_rng(3)
    q, k, v = rnd(1, 2, 12, 8, scale=2), rnd(1, 2, 12, 8, scale=2), rnd(1, 2, 12, 8)
    O0, l0 = oracle.attention(q, k, v, 0.5)
    O1, l1 = oracle.attention(q, k, v, 0.5, softcap=1e7)
    assert_close(O1, O0, 1e-9, "O")
    assert_close(l1, l0, 1e-9, "LSE")
    # weights through V = identity (D = Lk)
    L = 16
    q = (rng.standard_normal((1, 1, L, L)) * 50).astype(np.float32)
    k = (rng.standard_normal((1, 1, L, L)) * 50).astype(np.float32)
    eye = np.eye(L, dtype=np.float32)[None, None]
    W, _ = oracle.attention(q, k, eye, 1.0, softcap=1.5)
    assert np.allclose(W.sum(-1), 1.0, atol=1e-12)
    ratio = W.max(-1) / W.min(-1)
    assert np.all(ratio <= np.exp(2 * 1.5) * (1 + 1e-12))


def test_window_zero_is_the_diagonal():
    """Window (0, 0) leaves one key per row, j = p: O is that key's V row and
    LSE its own score."""
    q, k, v = rnd(1, 2, 9, 4), rnd(1, 2, 13, 4), rnd(1, 2, 13, 4)
    O, lse = oracle.attention(q, k, v, 0.5, window=(0, 0))
    p = np.arange(9) + 4
    assert np.array_equal(O, v[:, :, p, :].astype(np.float64))
    s = 0.5 * np.einsum("bhid,bhid->bhi", q.astype(np.float64), k[:, :, p, :].astype(np.float64))
    assert_close(lse, s, 1e-12, "LSE")


def test_window_equals_attention_on_the_key_slice():
    """A windowed row equals unmasked attention of that query over exactly the
    keys its window keeps (the oracle's own unwindowed path, pinned above)."""
    q, k, v = rnd(1, 1, 11, 8), rnd(1, 1, 30, 8), rnd(1, 1, 30, 8)
    for wl, wr in ((4, 2), (0, 5), (6, -1), (-1, 3)):
        O, lse = oracle.attention(q, k, v, 0.4, window=(wl, wr))
        for i in range(11):
            p = i + 19
            lo = 0 if wl < 0 else max(0, p - wl)
            hi = 30 if wr < 0 else min(30, p + wr + 1)
            Os, ls = oracle.attention(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi], 0.4)
            assert_close(O[0, 0, i], Os[0, 0, 0], 1e-14, "O row %d" % i)
            assert_close(lse[0, 0, i], ls[0, 0, 0], 1e-14, "LSE row %d" % i)


def test_window_unbounded_is_plain_and_causal():
    q, k, v = rnd(2, 2, 10, 8), rnd(2, 2, 14, 8), rnd(2, 2, 14, 8)
    O0, l0 = oracle.attention(q, k, v, 0.3)
    O1, l1 = oracle.attention(q, k, v, 0.3, window=(100, 100))
    assert np.array_equal(O0, O1) and np.array_equal(l0, l1)
    Oc, lc = oracle.attention(q, k, v, 0.3, causal=True)
    Ow, lw = oracle.attention(q, k, v, 0.3, window=(-1, 0))
    assert np.array_equal(Oc, Ow) and np.array_equal(lc, lw)


@pytest.mark.parametrize("case", BRUTE_CASES, ids=[str(i) for i in range(len(BRUTE_CASES))])
def test_brute_force(case):
    B, Hq, Hkv, Lq, Lk, D, scale, causal, bias_kind = case
    q, k, v = rnd(B, Hq, Lq, D, scale=2), rnd(B, Hkv, Lk, D, scale=2), rnd(B, Hkv, Lk, D)
    kw, bkw = {}, {}
    if bias_kind == "dense":
        bias = rnd(Hq, Lq, Lk)
        kw["bias"] = bias
        bkw["bias"] = bias[None]
    elif bias_kind == "dense_b":
        bias = rnd(B, 1, Lq, Lk)
        kw["bias"] = bias
        bkw["bias"] = bias
    elif bias_kind == "alibi":
        slopes = np.power(2.0, -8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        kw["alibi_slopes"] = slopes
        bkw["slopes"] = slopes
    O, lse = oracle.attention(q, k, v, scale, causal, **kw)
    Ob, lb = brute(q, k, v, scale, causal, **bkw)
    assert_close(O, Ob, 1e-12, "O")
    assert_close(lse, lb, 1e-12, "LSE")


def test_gqa_equals_repeated_mha():
    q, k, v = rnd(2, 8, 11, 16), rnd(2, 2, 19, 16), rnd(2, 2, 19, 16)
    a = oracle.attention(q, k, v, 0.3, True)
    b = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.3, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.attention(q, np.tile(k, (1, 4, 1, 1)), np.tile(v, (1, 4, 1, 1)), 0.3, True)
    assert np.max(np.abs(c[0] - a[0])) > 1e-2


def test_alibi_zero_slopes_is_no_bias():
    q, k, v = rnd(1, 4, 10, 8), rnd(1, 4, 14, 8), rnd(1, 4, 14, 8)
    a = oracle.attention(q, k, v, 0.5, True, alibi_slopes=np.zeros(4, np.float32))
    b = oracle.attention(q, k, v, 0.5, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_alibi_equals_dense_formula():
    Hq, Lq, Lk = 4, 10, 14
    q, k, v = rnd(1, Hq, Lq, 8), rnd(1, Hq, Lk, 8), rnd(1, Hq, Lk, 8)
    slopes = np.power(2.0, -8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
    pos = np.arange(Lq)[:, None] + (Lk - Lq)
    dense = (-slopes.astype(np.float64)[:, None, None] * np.abs(pos - np.arange(Lk)[None, :]))
    for causal in (False, True):
        a = oracle.attention(q, k, v, 0.5, causal, alibi_slopes=slopes)
        b = oracle.attention(q, k, v, 0.5, causal, bias=dense.astype(np.float32))
        assert_close(a[0], b[0], 1e-14, "O")
        assert_close(a[1], b[1], 1e-13, "LSE")


def test_large_logits_stay_finite():
    """q and K scaled by 40 (Mirage lecture section 5.5): logits in the
    thousands; an unstabilised exp overflows, the stable definition does not."""
    q, k, v = rnd(1, 2, 16, 8, scale=40), rnd(1, 2, 32, 8, scale=40), rnd(1, 2, 32, 8)
    O, lse = oracle.attention(q, k, v, 1.0, False)
    S = np.einsum("bhid,bhjd->bhij", q.astype(np.float64), k.astype(np.float64))
    assert np.max(np.abs(S)) > 700
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(S).sum(-1)
    assert not np.all(np.isfinite(naive))
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    Ob, lb = brute(q, k, v, 1.0, False)
    assert_close(O, Ob, 1e-12, "O")
    assert np.max(np.abs(lse - lb)) <= 1e-12 * np.max(np.abs(lb))


def test_row_subset_and_thread_count():
    q, k, v = rnd(2, 4, 21, 16), rnd(2, 2, 21, 16), rnd(2, 2, 21, 16)
    O, lse = oracle.attention(q, k, v, 0.25, True, threads=1)
    O8, lse8 = oracle.attention(q, k, v, 0.25, True, threads=8)
    assert np.array_equal(O, O8) and np.array_equal(lse, lse8)
    rows = [0, 5, 83, 2 * 4 * 21 - 1, 40]
    Os, ls = oracle.attention(q, k, v, 0.25, True, rows=rows)
    assert np.array_equal(Os, O.reshape(-1, 16)[rows])
    assert np.array_equal(ls, lse.reshape(-1)[rows])


# ----------------------------------------------------------------------------
# split-K combine
# ----------------------------------------------------------------------------
def partials_from_oracle(q, k, v, scale, bounds, shift_rng=None, lib=None):
    """(o_s, m_s, l_s) per chunk from the oracle on each key chunk:
    o_s = O_s, m_s = LSE_s, l_s = 1, optionally re-referenced to m_s + delta_s."""
    os_, ms, ls = [], [], []
    for a, b in bounds:
        O, lse = oracle.attention(q, k[:, :, a:b], v[:, :, a:b], scale, False, lib=lib)
        l = np.ones_like(lse)
        if shift_rng is not None:
            delta = shift_rng.uniform(-3, 3, size=lse.shape)
            fin = np.isfinite(lse)
            l = np.where(fin, np.exp(-delta), 0.0)
            O = O * np.where(fin, np.exp(-delta), 0.0)[..., None]
            lse = np.where(fin, lse + delta, lse)
        else:
            O = np.where(np.isfinite(lse)[..., None], O, 0.0)
            l = np.where(np.isfinite(lse), l, 0.0)
        os_.append(O)
        ms.append(lse)
        ls.append(l)
    return np.stack(os_, -2), np.stack(ms, -1), np.stack(ls, -1)


@pytest.mark.parametrize("bounds", [
    [(0, 128)],
    [(0, 64), (64, 128)],
    [(0, 32), (32, 64), (64, 96), (96, 128)],
    [(4 * s, 4 * s + 4) for s in range(32)],
    [(0, 50), (50, 51), (51, 128)],
    [(0, 70), (70, 70), (70, 128), (128, 128)],
])
def test_combine_equals_unsplit(bounds):
    q, k, v = rnd(2, 4, 1, 16, scale=2), rnd(2, 2, 128, 16, scale=2), rnd(2, 2, 128, 16)
    O, lse = oracle.attention(q, k, v, 0.3, False)
    for shift in (None, np.random.default_rng(7)):
        op, mp, lp = partials_from_oracle(q, k, v, 0.3, bounds, shift)
        Oc, lc = oracle.splitk_combine(op, mp, lp)
        assert_close(Oc, O, 1e-6, "O")   # partials pass through fp32
        assert_close(lc, lse, 1e-6, "LSE")


def test_combine_four_chunks_small_head():
    """1 query, 32 keys, head dim 8, four KV chunks (Mirage lecture section 5.5)."""
    q, k, v = rnd(1, 1, 1, 8), rnd(1, 1, 32, 8), rnd(1, 1, 32, 8)
    O, lse = oracle.attention(q, k, v, 1.0)
    op, mp, lp = partials_from_oracle(q, k, v, 1.0, [(8 * s, 8 * s + 8) for s in range(4)],
                                      np.random.default_rng(3))
    Oc, lc = oracle.splitk_combine(op, mp, lp)
    assert_close(Oc, O, 1e-6, "O")
    assert_close(lc, lse, 1e-6, "LSE")


def test_combine_all_empty_row():
    op = np.zeros((2, 3, 4), np.float32)
    mp = np.full((2, 3), -np.inf, np.float32)
    lp = np.zeros((2, 3), np.float32)
    Oc, lc = oracle.splitk_combine(op, mp, lp)
    assert np.all(Oc == 0.0) and np.all(np.isneginf(lc))


def test_combine_exact_weights():
    """Two chunks with m = (0, ln 3), l = 1: weights 1/4 and 3/4, LSE = ln 4."""
    op = np.array([[[4.0, 0.0], [0.0, 4.0]]], np.float32)
    mp = np.array([[0.0, math.log(3.0)]], np.float32)
    lp = np.ones((1, 2), np.float32)
    Oc, lc = oracle.splitk_combine(op, mp, lp)
    m1 = float(np.float32(math.log(3.0)))
    w1 = math.exp(m1) / (1 + math.exp(m1))
    assert_close(Oc.reshape(2), np.array([4 * (1 - w1), 4 * w1]), 1e-15, "O")
    assert abs(lc.item() - math.log(1 + math.exp(m1))) <= 1e-15


# ----------------------------------------------------------------------------
# backward: gradients of the forward definition
# ----------------------------------------------------------------------------
# The pages give the backward pass only by its shape (Twill review, section 7.2:
# one pass, five matrix products, one exponential); its values are the
# derivatives of the forward definition pinned above.  They are pinned here by
# central finite differences of the scipy brute force, sum(dO * O), which shares
# nothing with the oracle, and by invariants of the softmax.
BWD_CASES = [
    # B, Hq, Hkv, Lq, Lk, D, scale, causal, bias, softcap, window
    (1, 2, 1, 5, 7, 4, 0.5, True, None, 0.0, None),            # causal, Lq < Lk, GQA
    (1, 2, 2, 6, 6, 3, 0.7, False, "dense_inf", 0.0, None),    # dense bias with -inf entries and a dead row
    (2, 4, 2, 4, 9, 4, 0.4, False, "alibi", 0.0, (2, 1)),      # window, ALiBi
    (1, 3, 1, 5, 5, 4, 0.9, True, None, 1.5, None),            # strong soft cap, G = 3
    (1, 2, 1, 6, 4, 4, 0.6, True, None, 0.0, None),            # Lq > Lk: rows without keys
    (1, 2, 1, 5, 8, 4, 0.5, False, "dense", 2.0, (1, 0)),      # cap, window and dense bias
]


def _bwd_inputs(case, rng):
    B, Hq, Hkv, Lq, Lk, D, scale, causal, bias_kind, softcap, window = case
    q = rng.standard_normal((B, Hq, Lq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, Lk, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Lk, D)).astype(np.float32)
    do = rng.standard_normal((B, Hq, Lq, D)).astype(np.float32)
    kw, bkw = {"softcap": softcap, "window": window}, {"softcap": softcap, "window": window}
    if bias_kind in ("dense", "dense_inf"):
        bias = rng.standard_normal((B, Hq, Lq, Lk)).astype(np.float32)
        if bias_kind == "dense_inf":
            bias[:, :, 0, :] = -np.inf          # a row with no usable key
            bias[:, :, 1, 2] = -np.inf
            bias[:, 1, 3, ::2] = -np.inf
        kw["bias"] = bkw["bias"] = bias
    elif bias_kind == "alibi":
        slopes = np.power(2.0, -8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        kw["alibi_slopes"] = bkw["slopes"] = slopes
    return q, k, v, do, scale, causal, kw, bkw


def check_bwd_finite_differences(case, lib=None, elems=None, h=1e-5, tol=2e-7):
    """Every (or ``elems`` spread) element of dQ, dK, dV against the central
    difference of L = sum(dO * O) with O from the scipy brute force in fp64."""
    rng = np.random.default_rng(31)
    q, k, v, do, scale, causal, kw, bkw = _bwd_inputs(case, rng)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal, lib=lib, **kw)
    base = [np.asarray(x, np.float64) for x in (q, k, v)]
    dod = np.asarray(do, np.float64)

    def loss(arrs):
        O, _ = brute(arrs[0], arrs[1], arrs[2], scale, causal, **bkw)
        return float(np.sum(dod * O))

    for which, grad in enumerate((dq, dk, dv)):
        n = grad.size
        idx = range(n) if elems is None else np.linspace(0, n - 1, min(elems, n)).astype(int)
        for t in idx:
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[which].reshape(-1)[t] += h
            minus[which].reshape(-1)[t] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            got = grad.reshape(-1)[t]
            assert abs(got - fd) <= tol * max(1.0, abs(fd)), \
                "%s[%d]: oracle %.9f, finite difference %.9f" % ("qkv"[which], t, got, fd)


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(i) for i in range(len(BWD_CASES))])
def test_bwd_finite_differences(case):
    check_bwd_finite_differences(case)


def _visible_rows(B, Hq, Lq, Lk, causal, window):
    """[B, Hq, Lq] bool: the row sees at least one key."""
    pos = np.arange(Lq) + (Lk - Lq)
    lo = np.zeros(Lq, np.int64)
    hi = np.full(Lq, Lk, np.int64)
    if causal:
        hi = np.minimum(hi, pos + 1)
    if window is not None:
        if window[0] >= 0:
            lo = np.maximum(lo, pos - window[0])
        if window[1] >= 0:
            hi = np.minimum(hi, pos + window[1] + 1)
    return np.broadcast_to(hi > lo, (B, Hq, Lq))


@pytest.mark.parametrize("causal,window,alibi", [(False, None, False), (True, None, True),
                                                 (True, (5, -1), False), (False, (3, 2), True)])
def test_bwd_invariants(causal, window, alibi):
    """Without a cap: the value gradients of a K/V head add up to the output
    gradients of the rows that see a key (each softmax row sums to 1), and the
    key gradients add up to zero (a shift of every key by the same vector adds
    a constant to each score row, which the softmax ignores)."""
    rng = np.random.default_rng(41)
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 24, 40, 8
    q, k, v, do = (rng.standard_normal(s).astype(np.float32)
                   for s in ((B, Hq, Lq, D), (B, Hkv, Lk, D), (B, Hkv, Lk, D), (B, Hq, Lq, D)))
    kw = {"window": window}
    if alibi:
        kw["alibi_slopes"] = np.power(2.0, -np.arange(1, Hq + 1)).astype(np.float32)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.4, causal, **kw)
    vis = _visible_rows(B, Hq, Lq, Lk, causal, window)
    G = Hq // Hkv
    want = np.where(vis[..., None], do.astype(np.float64), 0.0).reshape(B, Hkv, G * Lq, D).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), want, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-10)
    assert np.all(dq[~vis] == 0.0)


def test_bwd_identical_keys_give_zero_dq():
    """All keys equal: every score of a row is the same function of q, so the
    weights do not depend on q (also under a cap, whose slope is then equal
    for all keys) and dQ = 0."""
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 2, 6, 8)).astype(np.float32)
    k = np.repeat(rng.standard_normal((1, 1, 1, 8)).astype(np.float32), 10, axis=2)
    v = rng.standard_normal((1, 1, 10, 8)).astype(np.float32)
    do = rng.standard_normal((1, 2, 6, 8)).astype(np.float32)
    for softcap in (0.0, 1.0):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, True, softcap=softcap)
        np.testing.assert_allclose(dq, 0.0, atol=1e-12)


def test_bwd_zero_q_value_gradient_closed_form():
    """Q = 0 and no bias: each row weighs its visible keys equally, so
    dV_j = sum over the rows i that see j of dO_i / (number of keys row i sees)."""
    rng = np.random.default_rng(47)
    Lq, Lk, D = 7, 11, 4
    q = np.zeros((1, 1, Lq, D), np.float32)
    k = rng.standard_normal((1, 1, Lk, D)).astype(np.float32)
    v = rng.standard_normal((1, 1, Lk, D)).astype(np.float32)
    do = rng.standard_normal((1, 1, Lq, D)).astype(np.float32)
    _, _, dv = oracle.attention_bwd(q, k, v, do, 1.0, True, window=(3, -1))
    want = np.zeros((Lk, D))
    for i in range(Lq):
        p = i + Lk - Lq
        keys = [j for j in range(Lk) if p - 3 <= j <= p]
        for j in keys:
            want[j] += do[0, 0, i].astype(np.float64) / len(keys)
    np.testing.assert_allclose(dv[0, 0], want, rtol=0, atol=1e-12)


def test_bwd_empty_shapes():
    rng = np.random.default_rng(53)
    q = rng.standard_normal((1, 2, 3, 4)).astype(np.float32)
    do = rng.standard_normal((1, 2, 3, 4)).astype(np.float32)
    k = np.zeros((1, 1, 0, 4), np.float32)
    dq, dk, dv = oracle.attention_bwd(q, k, k, do, 1.0, False)
    assert dq.shape == (1, 2, 3, 4) and np.all(dq == 0) and dk.shape == (1, 1, 0, 4)
    q0 = np.zeros((1, 2, 0, 4), np.float32)
    k1 = rng.standard_normal((1, 1, 5, 4)).astype(np.float32)
    dq, dk, dv = oracle.attention_bwd(q0, k1, k1, q0, 1.0, True)
    assert dq.shape == (1, 2, 0, 4) and np.all(dk == 0) and np.all(dv == 0)


def test_bwd_thread_count_does_not_matter():
    rng = np.random.default_rng(59)
    q, k, v, do = (rng.standard_normal(s).astype(np.float32)
                   for s in ((2, 4, 9, 8), (2, 2, 13, 8), (2, 2, 13, 8), (2, 4, 9, 8)))
    a = oracle.attention_bwd(q, k, v, do, 0.3, True, softcap=2.0, threads=1)
    b = oracle.attention_bwd(q, k, v, do, 0.3, True, softcap=2.0, threads=7)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ----------------------------------------------------------------------------
# row L2 norm (Neptune notes section 4 lists the numerically stable L2 norm
# among the reductions the repair algebra fuses): the plain definition
# ----------------------------------------------------------------------------
def _l2_strided(lib, x, stride):
    """call the oracle on rows `stride` floats apart (padding filled with 7s)"""
    import ctypes
    rows, H = x.shape
    buf = np.full((rows, stride), 7.0, np.float32)
    buf[:, :H] = x
    y = np.zeros((rows, H), np.float64)
    n = np.zeros((rows,), np.float64)
    rc = lib.oracle_l2norm(rows, H, buf.ctypes.data, stride, y.ctypes.data, n.ctypes.data)
    assert rc == 0
    return y, n


def check_l2norm_pins(lib=None):
    lib = lib or oracle.load()
    # 3-4-5 triangle, exact at any power-of-two scale (squares stay normal in fp64)
    for k in (0, 100, -120):
        x = np.array([[3.0 * 2.0 ** k, 4.0 * 2.0 ** k]], np.float32)
        y, n = oracle.l2norm(x, lib=lib)
        assert n[0] == 5.0 * 2.0 ** k, (k, n[0])
        assert y[0, 0] == 3.0 / 5.0 and y[0, 1] == 4.0 / 5.0
    # a row of ones has norm sqrt(H)
    for H in (1, 7, 4096):
        y, n = oracle.l2norm(np.ones((1, H), np.float32), lib=lib)
        assert n[0] == math.sqrt(H)
        assert np.all(np.abs(y - 1.0 / math.sqrt(H)) <= 1e-16)
    # zero row: norm 0, y = 0; one nonzero entry: y = +-1 there
    x = np.zeros((2, 9), np.float32)
    x[1, 4] = -2.5
    y, n = oracle.l2norm(x, lib=lib)
    assert n[0] == 0.0 and np.all(y[0] == 0.0)
    assert n[1] == 2.5 and y[1, 4] == -1.0 and np.count_nonzero(y[1]) == 1
    # scaling by 2^k scales the norm by 2^k exactly and leaves y unchanged
    rng = np.random.default_rng(61)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    y0, n0 = oracle.l2norm(x, lib=lib)
    for k in (60, -60):
        y1, n1 = oracle.l2norm((x * np.float32(2.0 ** k)).astype(np.float32), lib=lib)
        assert np.array_equal(n1, n0 * 2.0 ** k) and np.array_equal(y1, y0)
    # against numpy's norm on random rows of several magnitudes; unit rows
    x = (rng.standard_normal((6, 1000)) * np.array([1e-20, 1e-3, 1, 1e3, 1e15, 1e30])[:, None]).astype(np.float32)
    y, n = oracle.l2norm(x, lib=lib)
    ref = np.linalg.norm(x.astype(np.float64), axis=1)
    assert np.all(np.abs(n - ref) <= 1e-14 * ref)
    assert np.all(np.abs(np.sum(y * y, axis=1) - 1.0) <= 1e-13)
    # rows `stride` floats apart
    ys, ns = _l2_strided(lib, x, 1003)
    assert np.array_equal(ns, n) and np.array_equal(ys, y)


def test_l2norm_pins():
    check_l2norm_pins()


# ----------------------------------------------------------------------------
# planted mistakes must be caught
# ----------------------------------------------------------------------------
CAP_THEN_BIAS = """        if (J->softcap > 0.0) {
            const double th = tanh(sj / J->softcap);
            sj = J->softcap * th;
            slope = 1.0 - th * th;
        }
        if (J->bias_kind == ORACLE_BIAS_DENSE) {
            const int64_t *st = J->bias_strides;
            sj += (double)J->bias[b * st[0] + h * st[1] + i * st[2] + j * st[3]];
        } else if (J->bias_kind == ORACLE_BIAS_ALIBI) {
            double dist = (double)(p - j);
            if (dist < 0) dist = -dist;
            sj += -(double)J->slopes[h] * dist;
        }
"""
BIAS_THEN_CAP = """        if (J->bias_kind == ORACLE_BIAS_DENSE) {
            const int64_t *st = J->bias_strides;
            sj += (double)J->bias[b * st[0] + h * st[1] + i * st[2] + j * st[3]];
        } else if (J->bias_kind == ORACLE_BIAS_ALIBI) {
            double dist = (double)(p - j);
            if (dist < 0) dist = -dist;
            sj += -(double)J->slopes[h] * dist;
        }
        if (J->softcap > 0.0) {
            const double th = tanh(sj / J->softcap);
            sj = J->softcap * th;
            slope = 1.0 - th * th;
        }
"""

MUTANTS = {
    "kv_head_modulo": ("const int64_t hk = h / G;", "const int64_t hk = h % J->Hkv;"),
    "dropped_scale": ("double sj = J->scale * dot, slope = 1.0;", "double sj = dot, slope = 1.0;"),
    "alibi_sign": ("sj += -(double)J->slopes[h] * dist;", "sj += (double)J->slopes[h] * dist;"),
    "causal_off_by_one": ("if (J->causal && p + 1 < jhi) jhi = p + 1;", "if (J->causal && p < jhi) jhi = p;"),
    "softcap_undivided": ("const double th = tanh(sj / J->softcap);", "const double th = tanh(sj);"),
    "softcap_ignored": ("            sj = J->softcap * th;\n", "\n"),
    "softcap_after_bias": (CAP_THEN_BIAS, BIAS_THEN_CAP),
    "window_left_off_by_one": ("jlo = p - J->window_left;", "jlo = p - J->window_left + 1;"),
    "window_right_off_by_one": ("jhi = p + J->window_right + 1;", "jhi = p + J->window_right;"),
    "causal_top_left": ("const int64_t p = i + (J->Lk - J->Lq);", "const int64_t p = i;"),
    # backward
    "bwd_dropped_delta": ("const double dU = P * (dP - delta) * dc[j - jlo];",
                          "const double dU = P * dP * dc[j - jlo];"),
    "bwd_no_cap_slope": ("const double dU = P * (dP - delta) * dc[j - jlo];",
                         "const double dU = P * (dP - delta);"),
    "bwd_cap_slope_tanh": ("slope = 1.0 - th * th;", "slope = 1.0 - th;"),
    "bwd_dq_unscaled": ("dqrow[d] += J->scale * dU * (double)krow[d];", "dqrow[d] += dU * (double)krow[d];"),
    "bwd_dk_from_k": ("dkrow[d] += J->scale * dU * (double)qrow[d];",
                      "dkrow[d] += J->scale * dU * (double)krow[d];"),
    "bwd_dv_from_ds": ("dvrow[d] += P * (double)dorow[d];", "dvrow[d] += dU * (double)dorow[d];"),
    "bwd_delta_from_do": ("delta += (double)dorow[d] * orow[d];", "delta += (double)dorow[d] * (double)dorow[d];"),
    "bwd_heads_interleaved": ("for (int64_t h = hk * G; h < (hk + 1) * G; ++h) {",
                              "for (int64_t h = hk; h < J->Hq; h += J->Hkv) {"),
    "bwd_unnormalised_p": ("s[j - jlo] = exp(s[j - jlo] - m) / l;", "s[j - jlo] = exp(s[j - jlo] - m);"),
    # row L2 norm
    "l2_missing_sqrt": ("const double n = sqrt(ss);", "const double n = ss;"),
    "l2_sum_of_abs": ("ss += (double)xr[j] * (double)xr[j];", "ss += fabs((double)xr[j]);"),
    "l2_zero_row_nan": ("n > 0.0 ? (double)xr[j] / n : 0.0", "(double)xr[j] / n"),
    "l2_divides_by_square": ("n > 0.0 ? (double)xr[j] / n : 0.0", "n > 0.0 ? (double)xr[j] / (n * n) : 0.0"),
    "l2_stride_ignored": ("const float *xr = x + r * x_stride;", "const float *xr = x + r * H;"),
    "lse_log2": ("*lse = m + log(l);", "*lse = m + log2(l);"),
    "missing_normalise": ("for (int64_t d = 0; d < D; ++d) o[d] /= l;", ";"),
    "combine_weight_sign": ("const double w = exp(ms - M);", "const double w = exp(M - ms);"),
    "combine_unscaled_l": ("L += w * (double)l_part[r * S + s];", "L += (double)l_part[r * S + s];"),
    "dense_bias_transposed": ("sj += (double)J->bias[b * st[0] + h * st[1] + i * st[2] + j * st[3]];",
                              "sj += (double)J->bias[b * st[0] + h * st[1] + j * st[2] + i * st[3]];"),
}


def _pin_suite(lib):
    """A compact run of the pins above against library ``lib``; True if all pass."""
    try:
        for case in BRUTE_CASES:
            B, Hq, Hkv, Lq, Lk, D, scale, causal, bias_kind = case
            rng = np.random.default_rng(11)
            q = rng.standard_normal((B, Hq, Lq, D)).astype(np.float32)
            k = rng.standard_normal((B, Hkv, Lk, D)).astype(np.float32)
            v = rng.standard_normal((B, Hkv, Lk, D)).astype(np.float32)
            kw, bkw = {}, {}
            if bias_kind in ("dense", "dense_b"):
                bias = rng.standard_normal((B, Hq, Lq, Lk)).astype(np.float32)
                kw["bias"] = bkw["bias"] = bias
            elif bias_kind == "alibi":
                slopes = np.power(2.0, -8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
                kw["alibi_slopes"] = bkw["slopes"] = slopes
            O, lse = oracle.attention(q, k, v, scale, causal, lib=lib, **kw)
            Ob, lb = brute(q, k, v, scale, causal, **bkw)
            assert_close(O, Ob, 1e-12, "O")
            assert_close(lse, lb, 1e-12, "LSE")
        for case in MOD_CASES:
            q, k, v, scale, causal, kw, bkw = _mod_inputs(case, np.random.default_rng(23))
            O, lse = oracle.attention(q, k, v, scale, causal, lib=lib, **kw)
            Ob, lb = brute(q, k, v, scale, causal, **bkw)
            assert_close(O, Ob, 1e-12, "O")
            assert_close(lse, lb, 1e-12, "LSE")
        rng = np.random.default_rng(5)
        q = rng.standard_normal((1, 2, 1, 8)).astype(np.float32)
        k = rng.standard_normal((1, 2, 64, 8)).astype(np.float32)
        v = rng.standard_normal((1, 2, 64, 8)).astype(np.float32)
        O, lse = brute(q, k, v, 0.5)
        op, mp, lp = partials_from_oracle(q, k, v, 0.5, [(0, 20), (20, 64)], rng, lib=lib)
        Oc, lc = oracle.splitk_combine(op, mp, lp, lib=lib)
        assert_close(Oc, O, 1e-6, "combine O")
        assert_close(lc, lse, 1e-6, "combine LSE")
        for case in BWD_CASES:
            check_bwd_finite_differences(case, lib=lib, elems=12)
        check_l2norm_pins(lib)
    except AssertionError:
        return False
    return True


def test_pin_suite_accepts_oracle():
    assert _pin_suite(oracle.load())


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor not found: " + name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib_path = str(tmp_path / ("libmut_%s.so" % name))
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-o", lib_path,
                    str(path), "-lm"], check=True)
    assert not _pin_suite(oracle.load_path(lib_path)), "planted mistake not caught: " + name
