"""Streams, threads and graph capture (GPU).

Every entry point is stream-ordered and keeps no state between calls other
than a per-device count of compute units, so the same calls give bitwise the
same results whether they run one after another on one stream, at the same
time on two streams (from one host thread or from two), or replayed from a
captured HIP graph (the library enqueues kernels only: no memset or copy
nodes).  Streams use the default priority.
"""
import threading

import pytest
import torch

import synth
import online_softmax_fusion_amd as attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    attn.load_library()


def make_inputs(seed):
    w = synth.Workload("streams", 2, 4, 2, 300, 420, 128, "bf16", True, "alibi", seed)
    q, k, v = (t.cuda() for t in synth.make_qkv(w))
    wd = synth.Workload("streams-decode", 2, 8, 2, 1, 3000, 128, "bf16", False, "none", seed + 1)
    dq_, dk_, dv_ = (t.cuda() for t in synth.make_qkv(wd))
    x = synth.make_rows(synth.RowsWorkload("streams-rows", 64, 6144, "bf16", seed + 2)).cuda()
    return {"w": w, "q": q, "k": k, "v": v, "slopes": synth.alibi_slopes(4).cuda(),
            "do": synth.make_dout(w).cuda(), "dec": (dq_, dk_, dv_), "x": x}


def run_all(a):
    """Forward, backward, split-K decode and both row-norm paths of one input set."""
    s = a["w"].softmax_scale()
    o, lse = attn.attn_fwd_prefill(a["q"], a["k"], a["v"], s, True, alibi_slopes=a["slopes"])
    dq, dk, dv = attn.attn_bwd(a["q"], a["k"], a["v"], o, lse, a["do"], s, True, alibi_slopes=a["slopes"])
    od, lsed = attn.decode(*a["dec"], 7)
    y1, n1 = attn.l2norm_rows(a["x"], num_splits=1)
    y2, n2 = attn.l2norm_rows(a["x"], num_splits=5)
    return [o, lse, dq, dk, dv, od, lsed, y1, n1, y2, n2]


def assert_same(got, ref, what):
    for i, (g, r) in enumerate(zip(got, ref)):
        assert torch.equal(g, r), "%s: output %d differs" % (what, i)


def test_two_streams_match_one_stream():
    A, B = make_inputs(5001), make_inputs(5101)
    ref_a, ref_b = run_all(A), run_all(B)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(cur)
    s2.wait_stream(cur)
    for _ in range(3):
        with torch.cuda.stream(s1):
            got_a = run_all(A)
        with torch.cuda.stream(s2):
            got_b = run_all(B)
        cur.wait_stream(s1)
        cur.wait_stream(s2)
        torch.cuda.synchronize()
        assert_same(got_a, ref_a, "stream 1")
        assert_same(got_b, ref_b, "stream 2")


def test_two_host_threads():
    inputs = [make_inputs(5201), make_inputs(5301)]
    refs = [run_all(a) for a in inputs]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(st):
                for _ in range(4):
                    got = run_all(inputs[i])
                    st.synchronize()
                    assert_same(got, refs[i], "thread %d" % i)
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors[0]


def test_graph_replay_of_every_entry_point():
    """All calls of run_all captured in one graph; each of several replays,
    with eager work and synchronisations in between, equals the eager run."""
    A = make_inputs(5401)
    ref = run_all(A)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # warm the caching allocator outside the capture
        run_all(A)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run_all(A)
    for rep in range(3):
        for t in outs:
            t.fill_(0)   # a stale result cannot pass
        graph.replay()
        torch.cuda.synchronize()
        assert_same(outs, ref, "replay %d" % rep)
        run_all(make_inputs(5500 + rep))   # unrelated eager work between replays
        torch.cuda.synchronize()
