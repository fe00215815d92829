"""Benchmark of the fused attention forward on one MI355X.

Default run (N = 1):
  * prefill leg -- the causal bf16 workload B=4, H=32, L=4096, d=128; one step
    is one attn_fwd_prefill call over inputs already resident in HBM.  `value`
    is its throughput in algorithmic TFLOP/s (4 * d FLOP per visible
    query/key pair, masked pairs not counted).
  * the other prefill workloads, under "prefill_legs", each with its own
    roofline: ALiBi causal B=2, H=16, L=8192 (slopes formed in registers); the
    same problem with the ALiBi values given as a bf16 [H, L, L] bias tensor
    broadcast over the batch (the distinct bias bytes of the visible pairs,
    1.07 GB, take less time at the HBM peak than the matrix work at the bf16
    peak, so its roofline is the matrix cores', with the byte rate beside it);
    the long causal B=1, H=8, L=32768;
    the causal B=4, H=32, L=4096 with a soft cap of 50; the causal B=1, H=8,
    L=32768 with a sliding window of 4096 keys.
  * decode leg -- the split-K GQA workload B=16, Hq=32, Hkv=8, Lk=32768,
    d=128, 32 chunks of 1024 keys; one step is the local split-K kernel
    followed by the combine.  Reported under "decode" in algorithmic GB/s.
    The batch-1 decode (B=1, H=8, Lk=32768, split count chosen for the
    device) is reported the same way under "decode_b1"; its K/V copies are
    rotated so that each step reads from HBM, not from the 256 MB cache.
  * run metadata -- per leg the kernel's mean / p10 / p50 / p90 launch time
    and the graphics clock read from the driver's metrics while the leg ran
    ("sclk"); the GPU, its compute-unit and XCD counts and the host CPU model
    under "machine".  `--legs` runs a subset (for profiling runs).
  * roofline -- for the dominant kernel of each leg, algorithmic work per
    launch / the average launch duration measured with HIP events on the
    stream the kernel runs on.
  * backward leg -- attn_bwd (dQ kernel, then dK/dV kernel) on the shape the
    Twill review benchmarks the backward on (non-causal, B=4, H=32, d=128),
    at L=4096, with the forward's O and LSE as inputs.  Reported under
    "backward" in algorithmic TFLOP/s: 10 * d FLOP per visible pair (the five
    products S, dP, dV, dK, dQ), recomputation not counted.
  * plan leg -- attn_fwd (automatic choice of parallel dimensions) on a
    short-query GQA shape (B=1, Hq=32, Hkv=8, Lq=16, Lk=32768): the plan it
    picks, its time, and the prefill kernel's time on the same problem.
    Reported under "plan"; the same for a small-grid prefill with long rows
    (B=1, H=8, Lq=2048, Lk=32768, causal), where the plan splits the keys of
    the prefill kernel, under "plan_long_keys".  `--plan-sweep` times the
    three paths over the shape grid that set the planner's rule (one JSON
    line per shape).
  * l2norm leg -- the row L2 norm (the same repair algebra on a sum of
    squares): 32768 rows of 4096 bf16 values in one pass, and 8 rows of
    4194304 fp32 values split over the row.  Reported under "l2norm" in
    algorithmic GB/s (x read once, y and the norms written once).
  * cpu_baseline -- the fp64 oracle, timed on the host cores on a bounded
    sample of the prefill workload (whole heads), scaled to TFLOP/s.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E peak
METRIC = "prefill TFLOP/s (% MFMA peak); decode HBM GB/s (% of peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# algorithmic work (shared with the tests that pin these formulas)
# ----------------------------------------------------------------------------
def visible_pairs(Lq: int, Lk: int, causal: bool, window=None) -> int:
    """(query, key) pairs that enter the softmax for one head.  ``window`` =
    (left, right) keeps keys p - left <= j <= p + right (negative = unbounded)
    around each query's position p = i + Lk - Lq."""
    if window is not None:
        wl, wr = window
        total = 0
        for i in range(Lq):
            p = i + Lk - Lq
            lo, hi = 0, Lk - 1
            if causal:
                hi = min(hi, p)
            if wl >= 0:
                lo = max(lo, p - wl)
            if wr >= 0:
                hi = min(hi, p + wr)
            total += max(0, hi - lo + 1)
        return total
    if not causal:
        return Lq * Lk
    off = Lk - Lq
    total = 0
    # row i sees min(Lk, max(0, i + off + 1)) keys
    first_full = max(0, Lk - off - 1)          # rows i >= first_full see all Lk keys
    lo = max(0, -off)                          # rows below lo see nothing
    hi = min(Lq, first_full)
    if hi > lo:
        n = hi - lo
        a = lo + off + 1
        total += n * a + n * (n - 1) // 2
    if Lq > max(hi, lo):
        total += (Lq - max(hi, lo)) * Lk
    return total


def attention_flops(B, Hq, Lq, Lk, D, causal, window=None) -> int:
    """2*D FLOP for q.k and 2*D for p*v per visible pair."""
    return 4 * D * B * Hq * visible_pairs(Lq, Lk, causal, window)


def backward_flops(B, Hq, Lq, Lk, D, causal, window=None) -> int:
    """2*D FLOP for each of the five products (S, dP, dV, dK, dQ) per visible pair."""
    return 10 * D * B * Hq * visible_pairs(Lq, Lk, causal, window)


def prefill_bytes(B, Hq, Hkv, Lq, Lk, D, elem=2, o_elem=2) -> int:
    """Q, K, V read once; O and LSE written once."""
    return (B * Hq * Lq * D + 2 * B * Hkv * Lk * D) * elem + B * Hq * Lq * D * o_elem + B * Hq * Lq * 4


def decode_partial_kernel_bytes(B, Hq, Hkv, Lq, Lk, D, S, elem=2) -> int:
    """local split-K step: Q and K/V read once, partials (o, m, l) written once."""
    return (B * Hq * Lq * D + 2 * B * Hkv * Lk * D) * elem + B * Hq * Lq * S * (D + 2) * 4


def decode_step_bytes(B, Hq, Hkv, Lq, Lk, D, S, elem=2, o_elem=2) -> int:
    """whole decode: the local step, the partials read back, O and LSE written."""
    return (decode_partial_kernel_bytes(B, Hq, Hkv, Lq, Lk, D, S, elem) + B * Hq * Lq * S * (D + 2) * 4
            + B * Hq * Lq * D * o_elem + B * Hq * Lq * 4)


_TOKEN = re.compile(r'("(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\')|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed:
    what the compiler sees, so that a comment edit leaves the digest alone."""
    no_comments = _TOKEN.sub(lambda m: m.group(1) if m.group(1) is not None else " ", src)
    return " ".join(no_comments.split())


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ["online_softmax_fusion_amd/csrc/prefill_bf16.hip", "online_softmax_fusion_amd/csrc/attn_device.h"]
DECODE_SOURCES = ["online_softmax_fusion_amd/csrc/decode_bf16.hip", "online_softmax_fusion_amd/csrc/attn_device.h"]
BWD_SOURCES = ["online_softmax_fusion_amd/csrc/bwd_bf16.hip", "online_softmax_fusion_amd/csrc/attn_device.h"]
L2NORM_SOURCES = ["online_softmax_fusion_amd/csrc/l2norm.hip", "online_softmax_fusion_amd/csrc/attn_device.h"]


def measured_traffic(kernel: str, workload: str, sources) -> "int | None":
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    ent = table.get("%s @ %s" % (kernel, workload))
    if not ent or ent.get("source_digest") != source_digest(sources):
        return None
    return int(ent["traffic_bytes"])


def _sum_traffic(parts):
    """Total measured bytes per step of several kernels, or None if any is missing or stale."""
    total = 0
    for kernel, workload, sources in parts:
        t = measured_traffic(kernel, workload, sources)
        if t is None:
            return None
        total += t
    return total


# ----------------------------------------------------------------------------
# run metadata: GPU clock while a leg runs, host CPU model, percentiles
# ----------------------------------------------------------------------------
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _stats_ms(durs):
    """mean and percentiles of sorted per-launch durations (ms)."""
    n = len(durs)
    return {"mean": round(sum(durs) / n, 4), "p10": round(durs[n // 10], 4), "p50": round(durs[n // 2], 4),
            "p90": round(durs[(9 * n) // 10], 4)}


class ClockSampler:
    """The GPU's graphics clock while a leg runs: a background thread reads the
    driver's metrics table (amdsmi gpu_metrics, current clock of each XCD) every
    few milliseconds between start() and stop(), and stop() reports the median
    over the samples of the mean over XCDs.  The device is found by its PCI
    address.  Reports None (with the reason) where the metrics cannot be read;
    it never touches the GPU's settings."""

    _handle = None
    _why = None
    _lock = None

    def __init__(self, period_s=0.005):
        import threading

        self.period = period_s
        self.samples = []
        self.avg_samples = []
        self._stop = threading.Event()
        self._thread = None
        if ClockSampler._lock is None:
            ClockSampler._lock = threading.Lock()

    @classmethod
    def _open(cls):
        with cls._lock:
            if cls._handle is not None or cls._why is not None:
                return cls._handle
            try:
                import torch
                import amdsmi

                props = torch.cuda.get_device_properties(torch.cuda.current_device())
                want = "%04x:%02x:%02x" % (getattr(props, "pci_domain_id", 0), props.pci_bus_id,
                                           props.pci_device_id)
                amdsmi.amdsmi_init()
                handles = amdsmi.amdsmi_get_processor_handles()
                match = [h for h in handles if str(amdsmi.amdsmi_get_gpu_device_bdf(h)).lower().startswith(want)]
                if len(match) == 1:
                    cls._handle = match[0]
                elif len(handles) == 1:
                    cls._handle = handles[0]
                else:
                    cls._why = "no metrics device at PCI address %s" % want
            except Exception as e:   # metrics are optional: report why they are missing
                cls._why = "%s: %s" % (type(e).__name__, e)
            return cls._handle

    @staticmethod
    def _read(h):
        import amdsmi

        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        vals = [v for v in (m.get("current_gfxclks") or []) if isinstance(v, int) and 0 < v < 10000]
        if not vals and isinstance(m.get("current_gfxclk"), int):
            vals = [m["current_gfxclk"]]
        avg = m.get("average_gfxclk_frequency")
        stamp = m.get("firmware_timestamp")
        if not isinstance(stamp, int):
            stamp = m.get("system_clock_counter")
        return ((sum(vals) / len(vals) if vals else None), (avg if isinstance(avg, int) and 0 < avg < 10000 else None),
                stamp if isinstance(stamp, int) else None)

    def _run(self):
        # only tables the firmware wrote after the leg started count: the
        # driver refreshes them about once a second, so the first reads can
        # still describe the time before the leg
        h = self._open()
        first = None
        while h is not None and not self._stop.is_set():
            try:
                v, avg, stamp = self._read(h)
            except Exception:
                v = avg = stamp = None
            if first is None:
                first = stamp if stamp is not None else -1
            elif stamp is None or stamp != first:
                if v is not None:
                    self.samples.append(v)
                if avg is not None:
                    self.avg_samples.append(avg)
            self._stop.wait(self.period)

    def start(self):
        import threading

        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=2.0)
        if not self.samples:
            return {"mhz": None, "samples": 0,
                    "why": ClockSampler._why or "the metrics table was not refreshed while the leg ran"}
        x = sorted(self.samples)
        a = sorted(self.avg_samples)
        return {"mhz": round(x[len(x) // 2], 1), "min": round(x[0], 1), "max": round(x[-1], 1),
                "average_gfxclk_mhz": a[len(a) // 2] if a else None,
                "samples": len(x), "source": "amdsmi gpu_metrics current_gfxclks, mean over XCDs, median "
                                             "over the tables written while the leg's warm-up and timed "
                                             "steps ran"}


# ----------------------------------------------------------------------------
# legs
# ----------------------------------------------------------------------------
def warm_up(fn, warmup, seconds):
    """W untimed steps, continued until `seconds` of GPU work have run, so the
    timed steps start at settled clocks (the first second or so of work on an
    idle GPU runs measurably slower)."""
    import torch

    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def time_prefill(w, steps, warmup, warm_s=1.0):
    import torch
    import synth
    import online_softmax_fusion_amd as attn

    log("prefill leg: %s, generating inputs" % w.name)
    q, k, v = synth.make_qkv(w, device="cuda")
    kw = {"softcap": w.softcap, "window": w.window}
    if w.bias == "alibi":
        kw["alibi_slopes"] = synth.alibi_slopes(w.Hq).cuda()
    elif w.bias == "dense":
        kw["bias"] = synth.alibi_bias_tensor(w, "bf16", "cuda")   # [Hq, Lq, Lk], broadcast over B
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda")
    scale = w.softmax_scale()
    torch.cuda.synchronize()
    clock = ClockSampler().start()
    n = warm_up(lambda i: attn.attn_fwd_prefill(q, k, v, scale, w.causal, out=o, lse=lse, **kw), warmup, warm_s)
    log("prefill: %d untimed warm-up steps" % n)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        attn.attn_fwd_prefill(q, k, v, scale, w.causal, out=o, lse=lse, **kw)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = clock.stop()
    durs = sorted(a.elapsed_time(b) for a, b in ev)
    avg_ms = sum(durs) / len(durs)
    flops = attention_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, w.causal, w.window)
    log("prefill: wall %.3f ms/step, kernel avg %.4f ms (p10 %.4f, p90 %.4f), sclk %s MHz" %
        (wall * 1e3 / steps, avg_ms, durs[len(durs) // 10], durs[(9 * len(durs)) // 10], sclk.get("mhz")))
    del q, k, v, o, lse, kw
    torch.cuda.empty_cache()
    return {"step_s": wall / steps, "kern_s": avg_ms * 1e-3, "flops": flops, "durs": durs, "sclk": sclk}


def time_decode(w, steps, warmup, warm_s=1.0):
    """Decode step = split-K local step + combine, issued eagerly.  The kernel
    time comes from HIP events around the local step, timed over K launches of
    the local step alone issued back to back: at batch 1 the eager two-call
    step is bound by the host's launch work, and a kernel that starts after
    the GPU has idled runs slower than in steady use."""
    import torch
    import synth
    import online_softmax_fusion_amd as attn

    log("decode leg: %s, generating inputs" % w.name)
    q, k, v = synth.make_qkv(w, device="cuda")
    S = w.splits or attn.attn_decode_choose_splits(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, attn.attn_device_cu_count(0))
    kv_bytes = 2 * k.numel() * k.element_size()
    copies = max(1, math.ceil((512 << 20) / kv_bytes))     # keep the working set past the 256 MB cache
    kvs = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
    if copies > 1:
        log("decode: rotating %d K/V copies (%.0f MiB each)" % (copies, kv_bytes / 2 ** 20))
    op = torch.empty((w.B, w.Hq, w.Lq, S, w.D), dtype=torch.float32, device="cuda")
    mp = torch.empty((w.B, w.Hq, w.Lq, S), dtype=torch.float32, device="cuda")
    lp = torch.empty_like(mp)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda")
    scale = w.softmax_scale()

    def local(i, evs=None):
        kk, vv = kvs[i % copies]
        if evs:
            evs[0].record(torch.cuda.current_stream())
        attn.attn_fwd_decode_splitk(q, kk, vv, S, scale, w.causal, o_part=op, m_part=mp, l_part=lp)
        if evs:
            evs[1].record(torch.cuda.current_stream())

    def step(i):
        local(i)
        attn.attn_splitk_combine(op, mp, lp, out=o, lse=lse)

    torch.cuda.synchronize()
    clock = ClockSampler().start()
    n = warm_up(step, warmup, warm_s)
    log("decode: %d untimed warm-up steps" % n)
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        local(i, ev[i])
    torch.cuda.synchronize()
    sclk = clock.stop()
    durs = sorted(a.elapsed_time(b) for a, b in ev)
    avg_ms = sum(durs) / len(durs)

    # the same step as one attn_fwd call (the planner picks the same split-K
    # plan here; one binding call instead of two), with its workspace reused
    fwd_step_s = None
    plan = attn.attn_fwd_choose_plan(q, k, v, scale, w.causal)
    if plan.method == attn.ATTN_PLAN_SPLITK and plan.num_splits == S:
        wsb = torch.empty((plan.workspace_bytes,), dtype=torch.uint8, device="cuda")
        fstep = lambda i: attn.attn_fwd(q, kvs[i % copies][0], kvs[i % copies][1], scale, w.causal, out=o, lse=lse,
                                        workspace=wsb)
        warm_up(fstep, warmup, 0.2)
        t0 = time.perf_counter()
        for i in range(steps):
            fstep(i)
        torch.cuda.synchronize()
        fwd_step_s = (time.perf_counter() - t0) / steps
        del wsb

    # the same steps replayed from a HIP graph (one graph holds one step per
    # K/V copy), which removes the host launch cost between the two kernels
    graph_step_s = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(copies):
                step(i)
        reps = max(1, steps // copies)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_step_s = e0.elapsed_time(e1) * 1e-3 / (reps * copies)
        del g
    except RuntimeError as e:   # graph capture is an extra measurement; the eager step stands without it
        log("decode: graph replay not measured (%s)" % e)

    log("decode: %s S=%d, step %.4f ms (attn_fwd %s ms, graph replay %s ms), partial kernel avg %.4f ms "
        "(p10 %.4f, p90 %.4f)" %
        (w.name, S, wall * 1e3, "%.4f" % (fwd_step_s * 1e3) if fwd_step_s else "-",
         "%.4f" % (graph_step_s * 1e3) if graph_step_s else "-", avg_ms,
         durs[len(durs) // 10], durs[(9 * len(durs)) // 10]))
    del q, k, v, kvs, op, mp, lp, o, lse
    torch.cuda.empty_cache()
    return {"step_s": wall, "kern_s": avg_ms * 1e-3, "S": S, "durs": durs, "sclk": sclk, "copies": copies,
            "graph_step_s": graph_step_s, "fwd_step_s": fwd_step_s}


def time_backward(w, steps, warmup, warm_s=1.0):
    """One step = one attn_bwd call (both kernels) on resident inputs; the
    forward's O and LSE are computed once beforehand."""
    import torch
    import synth
    import online_softmax_fusion_amd as attn

    log("backward leg: %s, generating inputs" % w.name)
    q, k, v = synth.make_qkv(w, device="cuda")
    do = synth.make_dout(w, device="cuda")
    kw = {"softcap": w.softcap, "window": w.window}
    if w.bias == "alibi":
        kw["alibi_slopes"] = synth.alibi_slopes(w.Hq).cuda()
    scale = w.softmax_scale()
    o, lse = attn.attn_fwd_prefill(q, k, v, scale, w.causal, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((attn.attn_bwd_workspace_bytes(w.B, w.Hq, w.Lq),), dtype=torch.uint8, device="cuda")

    def step(i, evs=None):
        if evs:
            evs[0].record(torch.cuda.current_stream())
        attn.attn_bwd(q, k, v, o, lse, do, scale, w.causal, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
        if evs:
            evs[1].record(torch.cuda.current_stream())

    n = warm_up(step, warmup, warm_s)
    log("backward: %d untimed warm-up steps" % n)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    durs = sorted(a.elapsed_time(b) for a, b in ev)
    avg_ms = sum(durs) / len(durs)
    flops = backward_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, w.causal, w.window)
    log("backward: step %.4f ms, kernels avg %.4f ms (p10 %.4f, p90 %.4f)" %
        (wall * 1e3, avg_ms, durs[len(durs) // 10], durs[(9 * len(durs)) // 10]))
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return wall, avg_ms * 1e-3, flops


def _median_us(fn, reps=10):
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    d = sorted(a.elapsed_time(b) for a, b in ev)
    return d[len(d) // 2] * 1e3


def l2norm_bytes(rows, H, elem_x, elem_y) -> int:
    """x read once, y written once, one fp32 norm per row."""
    return rows * H * (elem_x + elem_y) + rows * 4


def time_l2norm(w, steps, warmup, warm_s=1.0):
    """One step = one l2norm_rows call (one or two kernels) on resident rows."""
    import torch
    import synth
    import online_softmax_fusion_amd as attn

    x = synth.make_rows(w, device="cuda")
    S = attn.l2norm_choose_splits(w.rows, w.H, x.dtype, attn.attn_device_cu_count(0))
    y = torch.empty_like(x)
    n = torch.empty((w.rows,), dtype=torch.float32, device="cuda")
    ws = torch.empty((max(attn.l2norm_workspace_bytes(w.rows, S), 16),), dtype=torch.uint8, device="cuda")

    def step(i, evs=None):
        if evs:
            evs[0].record(torch.cuda.current_stream())
        attn.l2norm_rows(x, out=y, norm=n, num_splits=S, workspace=ws)
        if evs:
            evs[1].record(torch.cuda.current_stream())

    warm_up(step, warmup, warm_s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) for a, b in ev)
    avg_s = sum(durs) / len(durs) * 1e-3
    e = x.element_size()
    alg = l2norm_bytes(w.rows, w.H, e, e)
    gbs = alg / avg_s / 1e9
    log("l2norm: %s S=%d, %.4f ms, %.0f GB/s" % (w.name, S, avg_s * 1e3, gbs))
    del x, y, n, ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "splits": S, "ms_per_step": round(avg_s * 1e3, 4), "value": round(gbs, 1),
            "unit": "GB/s", "algorithmic_bytes": alg,
            "roofline": {"kernel": "l2norm_onepass_kernel" if S == 1 else "l2norm_partial_kernel + l2norm_scale_kernel",
                         "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": _sum_traffic([("l2norm_onepass_kernel", w.name, L2NORM_SOURCES)] if S == 1 else
                                                 [("l2norm_partial_kernel", w.name, L2NORM_SOURCES),
                                                  ("l2norm_scale_kernel", w.name, L2NORM_SOURCES)])}}


def time_plan(w):
    """attn_fwd with its plan against the prefill kernel on the same problem."""
    import torch
    import synth
    import online_softmax_fusion_amd as attn

    q, k, v = synth.make_qkv(w, device="cuda")
    sc = w.softmax_scale()
    plan = attn.attn_fwd_choose_plan(q, k, v, sc, w.causal)
    ws = torch.empty((max(plan.workspace_bytes, 16),), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda")
    t_fwd = _median_us(lambda: attn.attn_fwd(q, k, v, sc, w.causal, out=o, lse=lse, workspace=ws), 20)
    t_pf = _median_us(lambda: attn.attn_fwd_prefill(q, k, v, sc, w.causal, out=o, lse=lse), 20)
    method = {attn.ATTN_PLAN_SPLITK: "splitk", attn.ATTN_PLAN_PREFILL_SPLIT: "split_prefill"}.get(plan.method,
                                                                                                "prefill")
    log("plan: %s -> %s S=%d, %.1f us (prefill kernel %.1f us)" % (w.name, method, plan.num_splits, t_fwd, t_pf))
    return {"workload": w.name, "method": method,
            "splits": plan.num_splits, "attn_fwd_us": round(t_fwd, 1), "prefill_kernel_us": round(t_pf, 1),
            "speedup": round(t_pf / t_fwd, 2)}


def plan_sweep(causal):
    """The forward paths over B 1, 4; Hq/Hkv 8/8, 32/8, 64/8; Lq 1..2048;
    Lk 4096, 32768 (d = 128, bf16): prefill kernel, split-K at each split
    count, the prefill kernel over key chunks at each chunk count, the
    planner's choice.  One JSON line per shape on stdout."""
    import torch
    import synth
    import online_softmax_fusion_amd as attn

    cu = attn.attn_device_cu_count(0)
    for Lk in (4096, 32768):
        for B in (1, 4):
            for Hq, Hkv in ((8, 8), (32, 8), (64, 8)):
                w = synth.Workload("sweep", B, Hq, Hkv, 1, Lk, 128, "bf16", causal, "none", 5)
                _, k, v = synth.make_qkv(w, device="cuda")
                for Lq in (1, 4, 16, 64, 128, 256, 512, 1024, 2048):
                    q = synth.normal((B, Hq, Lq, 128), 5, 0, "bf16", "cuda")
                    sc = w.softmax_scale()
                    o = torch.empty_like(q)
                    lse = torch.empty((B, Hq, Lq), device="cuda")
                    res = {"B": B, "Hq": Hq, "Hkv": Hkv, "Lq": Lq, "Lk": Lk, "causal": causal,
                           "prefill_us": round(_median_us(lambda: attn.attn_fwd_prefill(q, k, v, sc, causal, out=o,
                                                                                       lse=lse)), 1)}
                    blocks = B * Hkv * ((Hq // Hkv * Lq + 31) // 32)
                    best = None
                    for S in (1, 2, 4, 8, 16, 32, 64, 128):
                        if S > max(1, Lk // 256) or (S > 1 and blocks * S > 8 * cu):
                            continue
                        op = torch.empty((B, Hq, Lq, S, 128), device="cuda")
                        mp = torch.empty((B, Hq, Lq, S), device="cuda")
                        lp = torch.empty_like(mp)

                        def run():
                            attn.attn_fwd_decode_splitk(q, k, v, S, sc, causal, o_part=op, m_part=mp, l_part=lp)
                            attn.attn_splitk_combine(op, mp, lp, out=o, lse=lse)

                        t = _median_us(run)
                        res["splitk_S%d_us" % S] = round(t, 1)
                        if best is None or t < best[1]:
                            best = (S, t)
                    res["best_S"], res["best_splitk_us"] = best[0], round(best[1], 1)
                    # the prefill kernel over key chunks, then the combine
                    pblocks = B * Hq * ((Lq + 127) // 128)
                    pbest = None
                    for S in (2, 4, 8, 16, 32):
                        if S > Lk // 512 or pblocks * (S // 2) > 2 * cu:
                            continue
                        op = torch.empty((B, Hq, Lq, S, 128), device="cuda")
                        mp = torch.empty((B, Hq, Lq, S), device="cuda")
                        lp = torch.empty_like(mp)

                        def run_p():
                            attn.attn_fwd_prefill_splitk(q, k, v, S, sc, causal, o_part=op, m_part=mp, l_part=lp)
                            attn.attn_splitk_combine(op, mp, lp, out=o, lse=lse)

                        t = _median_us(run_p)
                        res["psplit_S%d_us" % S] = round(t, 1)
                        if pbest is None or t < pbest[1]:
                            pbest = (S, t)
                    if pbest is not None:
                        res["best_pS"], res["best_psplit_us"] = pbest[0], round(pbest[1], 1)
                    plan = attn.attn_fwd_choose_plan(q, k, v, sc, causal)
                    res["plan"] = {attn.ATTN_PLAN_SPLITK: "splitk", attn.ATTN_PLAN_PREFILL_SPLIT: "psplit"}.get(
                        plan.method, "prefill")
                    res["plan_S"] = plan.num_splits
                    print(json.dumps(res), flush=True)
                del k, v
                torch.cuda.empty_cache()


def cpu_baseline(w, budget_s=15.0):
    """The fp64 oracle as it stands, on whole heads of the prefill workload."""
    import numpy as np
    import synth
    import oracle

    threads = oracle.default_threads()
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        threads = max(1, min(threads, int(env)))
    G = w.Hq // w.Hkv

    def run(n_heads):
        ws = w.with_(B=1, Hq=n_heads * G, Hkv=n_heads)   # n K/V heads with their query groups
        q, k, v = synth.make_qkv(ws)
        q, k, v = q.float().numpy(), k.float().numpy(), v.float().numpy()
        t0 = time.perf_counter()
        oracle.attention(q, k, v, w.softmax_scale(), w.causal, softcap=w.softcap, window=w.window,
                         threads=threads)
        t = time.perf_counter() - t0
        return t, attention_flops(1, n_heads * G, w.Lq, w.Lk, w.D, w.causal, w.window)

    t1, f1 = run(1)
    n = int(max(1, min(w.B * w.Hkv, round(budget_s / max(t1, 1e-3)))))
    if n > 1:
        t1, f1 = run(n)
    log("cpu baseline: %d head(s) in %.2f s on %d threads" % (n, t1, threads))
    return {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d whole K/V head(s) with their %d query head(s) each (%d query rows x %d keys%s, "
                      "d=%d), drawn with the workload's recipe, of %s; fp64; %.1f s" %
                      (n, G, w.Lq, w.Lk, ", causal" if w.causal else "", w.D, w.name, t1)}


def _counter_kib(csv_path, counter, kernel_substr, grid=None):
    """Mean value of `counter` (KiB) over the dispatches whose kernel name
    contains `kernel_substr` (a string, or a tuple of strings that must all
    appear) (and, if given, whose grid has `grid` work-items:
    the bench launches some kernels on more than one shape) in a rocprofv3
    counter_collection.csv."""
    import csv

    parts = (kernel_substr,) if isinstance(kernel_substr, str) else tuple(kernel_substr)
    vals = []
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and all(x in row["Kernel_Name"] for x in parts) and \
                    (grid is None or int(row["Grid_Size"]) == grid):
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise ValueError("no %s samples for %s in %s" % (counter, kernel_substr, csv_path))
    return sum(vals) / len(vals)


def traffic_table(d):
    """HBM bytes per launch of the kernels a default bench run times, from
    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by what the same
    counters read for a plain device copy of known size.  Under `d`: fetch/
    and write/ (a default bench run), fetch_b1/ and write_b1/ (a run of the
    decode_b1 leg alone, whose decode grid the plan leg shares), cfetch/ and
    cwrite/ (the copy)."""
    import glob
    import synth
    import online_softmax_fusion_amd as attn

    def csv_of(sub):
        hits = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not hits:
            raise FileNotFoundError("no counter_collection.csv under %s" % os.path.join(d, sub))
        return hits[0]

    copy_bytes = 1 << 30
    cf = _counter_kib(csv_of("cfetch"), "FETCH_SIZE", "copyBuffer")
    cw = _counter_kib(csv_of("cwrite"), "WRITE_SIZE", "copyBuffer")
    fscale, wscale = copy_bytes / 1024.0 / cf, copy_bytes / 1024.0 / cw
    out = {"_about": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per "
                     "dispatch, mean over the dispatches of the run), each scaled by the factor that makes the "
                     "same counter read the known size of a plain 1 GiB device copy (bench.py "
                     "--copy-calibration). Keys are 'kernel @ workload'. source_digest ties an entry to the "
                     "kernel source it was measured on (comments and whitespace aside); "
                     "bench.py reports null traffic once that source changes.",
           "calibration": {"copy_bytes": copy_bytes, "fetch_kib_per_copy": cf, "write_kib_per_copy": cw,
                           "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5)}}
    wp, wd, wbk, wl, wll = synth.C2_CAUSAL, synth.C4_DECODE, synth.BWD_PREFILL, synth.L2N_ROWS, synth.L2N_LONG
    w3, w3d, w5, w5d = synth.C3_ALIBI, synth.C3_DENSE, synth.C5_PREFILL, synth.C5_DECODE
    wsc, wwin = synth.SOFTCAP_PREFILL, synth.WINDOW_PREFILL
    S = wd.splits
    S5 = attn.attn_decode_choose_splits(w5d.B, w5d.Hq, w5d.Hkv, w5d.Lq, w5d.Lk, 256)
    Sl = 128                                        # l2norm_choose_splits for the long rows on 256 CUs
    q_e = wbk.B * wbk.Hq * wbk.Lq * wbk.D * 2           # one [B, Hq, L, D] bf16 tensor
    kv_e = wbk.B * wbk.Hkv * wbk.Lk * wbk.D * 2
    rows4 = wbk.B * wbk.Hq * wbk.Lq * 4                # one fp32 value per query row

    def pf(w):
        return prefill_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D)

    def pgrid(w):   # 64 work-items per 32 query rows, whatever the wave count
        return (w.Lq // 32) * 64 * w.B * w.Hq

    entries = [
        # kernel, name match, workload, sources, algorithmic bytes, grid work-items, counter runs
        # (the C2 entry names its 4-wave form: the backward leg's non-causal forward runs the
        # 8-wave form on the same grid; the template's third argument is the score modifier:
        # 0 none, 10 causal ALiBi folded into the scores, 9 dense bf16 bias loaded in tiles)
        ("prefill_bf16_kernel", ("prefill_bf16_kernel<128, 4, 0, true>",), wp, PREFILL_SOURCES, pf(wp), pgrid(wp),
         ""),
        ("prefill_bf16_kernel", ("prefill_bf16_kernel<128, ", ", 10, true>"), w3, PREFILL_SOURCES, pf(w3), pgrid(w3),
         ""),
        ("prefill_bf16_kernel", ("prefill_bf16_kernel<128, 8, 12, true>",), w3d, PREFILL_SOURCES,
         pf(w3d) + dense_bias_bytes(w3d), pgrid(w3d), ""),
        ("prefill_bf16_kernel", ("prefill_bf16_kernel<128, 8, 0, true>",), w5, PREFILL_SOURCES, pf(w5), pgrid(w5),
         ""),
        # soft cap 50 (11: the soft cap for caps up to 64) and the sliding window (four waves, kind 0,
        # on the long causal grid)
        ("prefill_bf16_kernel", ("prefill_bf16_kernel<128, 4, 11, true>",), wsc, PREFILL_SOURCES, pf(wsc),
         pgrid(wsc), ""),
        ("prefill_bf16_kernel", ("prefill_bf16_kernel<128, 4, 0, true>",), wwin, PREFILL_SOURCES, pf(wwin),
         pgrid(wwin), ""),
        ("decode_bf16_kernel", ("decode_bf16_kernel",), wd, DECODE_SOURCES,
         decode_partial_kernel_bytes(wd.B, wd.Hq, wd.Hkv, wd.Lq, wd.Lk, wd.D, S), S * wd.B * wd.Hkv * 256, ""),
        ("decode_bf16_kernel", ("decode_bf16_kernel",), w5d, DECODE_SOURCES,
         decode_partial_kernel_bytes(w5d.B, w5d.Hq, w5d.Hkv, w5d.Lq, w5d.Lk, w5d.D, S5), None, "_b1"),
        # dQ: reads Q, dO, O, LSE, K, V; writes dQ, Delta, LSE*log2(e)
        ("bwd_dq_kernel", ("bwd_dq_kernel",), wbk, BWD_SOURCES, 4 * q_e + rows4 + 2 * kv_e + 2 * rows4,
         (wbk.Lq // 128) * wbk.B * wbk.Hq * 256, ""),
        # dK/dV (the paired-wave kernel at d = 128): reads Q, dO, Delta, LSE*log2(e), K, V; writes dK, dV
        ("bwd_dkdv_pair_kernel", ("bwd_dkdv_pair_kernel",), wbk, BWD_SOURCES, 2 * q_e + 2 * rows4 + 4 * kv_e,
         (wbk.Lk // 128) * wbk.B * wbk.Hkv * 512, ""),
        ("l2norm_onepass_kernel", ("l2norm_onepass_kernel",), wl, L2NORM_SOURCES, l2norm_bytes(wl.rows, wl.H, 2, 2),
         (wl.rows // 4) * 256, ""),
        # split path: the partial kernel reads x and writes one partial per chunk; the scale kernel
        # reads the partials and x and writes y and the norms
        ("l2norm_partial_kernel", ("l2norm_partial_kernel",), wll, L2NORM_SOURCES,
         wll.rows * wll.H * 4 + wll.rows * Sl * 8, wll.rows * Sl * 256, ""),
        ("l2norm_scale_kernel", ("l2norm_scale_kernel",), wll, L2NORM_SOURCES,
         wll.rows * wll.H * 8 + wll.rows * Sl * 8 + wll.rows * 4, wll.rows * Sl * 256, ""),
    ]
    for kernel, match, w, srcs, alg, grid, run in entries:
        try:
            fk = _counter_kib(csv_of("fetch" + run), "FETCH_SIZE", match, grid)
            wk = _counter_kib(csv_of("write" + run), "WRITE_SIZE", match, grid)
        except (ValueError, FileNotFoundError):
            continue
        fb, wbytes = int(round(fk * 1024 * fscale)), int(round(wk * 1024 * wscale))
        out["%s @ %s" % (kernel, w.name)] = {
            "kernel": kernel, "workload": w.name, "grid_work_items": grid, "source_digest": source_digest(srcs),
            "fetch_kib": round(fk, 1), "write_kib": round(wk, 1), "fetch_bytes": fb, "write_bytes": wbytes,
            "traffic_bytes": fb + wbytes, "algorithmic_bytes": alg,
            "traffic_over_algorithmic": round((fb + wbytes) / alg, 4)}
    return out


ALL_LEGS = ("prefill", "prefill_c3", "prefill_c3_dense", "prefill_c5", "prefill_softcap", "prefill_window", "decode",
            "decode_b1", "plan", "l2norm", "backward")


def dense_bias_bytes(w, elem=2) -> int:
    """distinct bias elements of the visible pairs: the bench's bias is one
    [Hq, Lq, Lk] tensor shared by the batch, so each is read once."""
    return w.Hq * visible_pairs(w.Lq, w.Lk, w.causal, w.window) * elem


def prefill_leg_json(w, r):
    """One prefill leg: whole-step throughput, kernel percentiles, and the
    roofline of prefill_bf16_kernel (matrix-core bound; with a dense bias the
    bias bytes make it bound by HBM, and both fractions are given)."""
    flops = r["flops"]
    kern_tf = flops / r["kern_s"] / 1e12
    leg = {"workload": w.name, "bias": w.bias, "softcap": w.softcap, "window": list(w.window) if w.window else None,
           "seed": w.seed, "value": round(flops / r["step_s"] / 1e12, 2),
           "unit": "TFLOP/s",
           "ms_per_step": round(r["step_s"] * 1e3, 4), "kernel_ms": _stats_ms(r["durs"]), "sclk": r["sclk"]}
    traffic = measured_traffic("prefill_bf16_kernel", w.name, PREFILL_SOURCES)
    if w.bias == "dense":
        # the bound is whichever roofline time is longer: the algorithmic bytes
        # (Q, K, V, the distinct bias bytes, O, LSE) at the HBM peak or the
        # matrix work at the bf16 peak; the other rate is given beside it
        nbytes = prefill_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D) + dense_bias_bytes(w)
        gbs = nbytes / r["kern_s"] / 1e9
        hbm_bound = nbytes / (HBM_PEAK_GBS * 1e9) > flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        if hbm_bound:
            leg["roofline"] = {"kernel": "prefill_bf16_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                               "traffic": traffic, "algorithmic_bytes": nbytes,
                               "mfma_achieved_tflops": round(kern_tf, 2),
                               "mfma_frac": round(kern_tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            leg["roofline"] = {"kernel": "prefill_bf16_kernel", "bound": "mfma", "achieved": round(kern_tf, 2),
                               "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(kern_tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                               "algorithmic_bytes": nbytes, "hbm_achieved_gbs": round(gbs, 1),
                               "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        leg["roofline"] = {"kernel": "prefill_bf16_kernel", "bound": "mfma", "achieved": round(kern_tf, 2),
                           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(kern_tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    return leg


def decode_leg_json(w, r):
    """One decode leg: the whole step (local split-K step + combine) in
    algorithmic GB/s, and the roofline of the local step's kernel."""
    S = r["S"]
    d_bytes = decode_step_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, S)
    k_bytes = decode_partial_kernel_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, S)
    gbs = d_bytes / r["step_s"] / 1e9
    kgbs = k_bytes / r["kern_s"] / 1e9
    gs = r.get("graph_step_s")
    return {"workload": w.name, "seed": w.seed, "splits": S, "kv_copies_rotated": r["copies"], "value": round(gbs, 1),
            "unit": "GB/s", "ms_per_step": round(r["step_s"] * 1e3, 4),
            "graph_replay": None if not gs else {"ms_per_step": round(gs * 1e3, 4),
                                                 "value": round(d_bytes / gs / 1e9, 1), "unit": "GB/s"},
            "attn_fwd_step": None if not r.get("fwd_step_s") else {
                "ms_per_step": round(r["fwd_step_s"] * 1e3, 4), "value": round(d_bytes / r["fwd_step_s"] / 1e9, 1),
                "unit": "GB/s"},
            "kernel_ms": _stats_ms(r["durs"]),
            "sclk": r["sclk"],
            "roofline": {"kernel": "decode_bf16_kernel", "bound": "hbm", "achieved": round(kgbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_bf16_kernel", w.name, DECODE_SOURCES)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=2.0,
                    help="keep warming up (untimed) until this much time has passed")
    ap.add_argument("--prefill", default=None, help="prefill workload name (default: causal B4 H32 L4096)")
    ap.add_argument("--decode", default=None, help="decode workload name (default: GQA B16 Lk32768)")
    ap.add_argument("--splits", type=int, default=None, help="override the decode split count")
    ap.add_argument("--backward", default=None,
                    help="backward workload name (default: non-causal B4 H32 L4096), or 'none' to skip")
    ap.add_argument("--legs", default="all",
                    help="comma-separated subset of %s (default: all; the headline needs 'prefill')" %
                         ",".join(ALL_LEGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--plan-sweep", choices=("causal", "noncausal"), default=None,
                    help="only time both forward paths over the planner's shape grid (JSON lines)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work to time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--traffic-table", metavar="DIR", default=None,
                    help="only summarise the rocprofv3 FETCH_SIZE / WRITE_SIZE runs under DIR (fetch/, write/, "
                         "cfetch/, cwrite/) into the per-kernel traffic table, printed as JSON")
    args = ap.parse_args()
    if args.traffic_table:
        print(json.dumps(traffic_table(args.traffic_table), indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requested %d)" %
              max(args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("steps must be >= 1 and warmup >= 0")

    import torch
    import synth
    import online_softmax_fusion_amd as attn

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_calibration:
        n = 256 << 20
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "dispatches": 3}))
        return
    attn.load_library()
    if args.plan_sweep:
        plan_sweep(args.plan_sweep == "causal")
        return
    wp = synth.WORKLOADS[args.prefill] if args.prefill else synth.C2_CAUSAL
    wd = synth.WORKLOADS[args.decode] if args.decode else synth.C4_DECODE
    if args.splits:
        wd = wd.with_(splits=args.splits)
    legs = set(ALL_LEGS if args.legs == "all" else args.legs.split(","))
    unknown = legs - set(ALL_LEGS)
    if unknown:
        sys.exit("unknown legs: %s (known: %s)" % (",".join(sorted(unknown)), ",".join(ALL_LEGS)))
    if args.backward == "none":
        legs.discard("backward")
    wb = synth.WORKLOADS[args.backward] if args.backward not in (None, "none") else synth.BWD_PREFILL

    torch.cuda.synchronize()
    result = {
        "metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16 inputs)",
        "config": {"workload": wp.name, "seed": wp.seed, "B": wp.B, "H": wp.Hq, "Lq": wp.Lq, "Lk": wp.Lk, "D": wp.D,
                   "causal": wp.causal, "bias": wp.bias, "softcap": wp.softcap,
                   "window": list(wp.window) if wp.window else None, "parallelism": "single GPU"},
    }
    props = torch.cuda.get_device_properties(0)
    result["machine"] = {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
                         "compute_units": attn.attn_device_cu_count(0), "xcds": attn.attn_device_xcd_count(0),
                         "cpu_model": cpu_model(), "host_threads": os.cpu_count()}
    if "prefill" in legs:
        r = time_prefill(wp, args.steps, args.warmup, args.warm_seconds)
        leg = prefill_leg_json(wp, r)
        result["value"] = leg["value"]
        result["ms_per_step"] = leg["ms_per_step"]
        result["roofline"] = leg["roofline"]
        result["kernel_ms"] = leg["kernel_ms"]
        result["sclk"] = leg["sclk"]
    extra = [("prefill_c3", synth.C3_ALIBI), ("prefill_c3_dense", synth.C3_DENSE), ("prefill_c5", synth.C5_PREFILL),
             ("prefill_softcap", synth.SOFTCAP_PREFILL), ("prefill_window", synth.WINDOW_PREFILL)]
    pl = [prefill_leg_json(w, time_prefill(w, args.steps, args.warmup, args.warm_seconds))
          for name, w in extra if name in legs]
    if pl:
        result["prefill_legs"] = pl
    if "decode" in legs:
        result["decode"] = decode_leg_json(wd, time_decode(wd, args.steps, args.warmup, args.warm_seconds))
    if "decode_b1" in legs:
        result["decode_b1"] = decode_leg_json(synth.C5_DECODE, time_decode(synth.C5_DECODE, args.steps, args.warmup,
                                                                           args.warm_seconds))
    if "plan" in legs:
        result["plan"] = time_plan(synth.PLAN_SHORT_GQA)
        result["plan_long_keys"] = time_plan(synth.PLAN_LONG_KEYS)
    if "l2norm" in legs:
        result["l2norm"] = [time_l2norm(w, args.steps, args.warmup, args.warm_seconds)
                            for w in (synth.L2N_ROWS, synth.L2N_LONG)]
    if "backward" in legs:
        b_step_s, b_kern_s, b_flops = time_backward(wb, args.steps, args.warmup, args.warm_seconds)
        b_kern_tflops = b_flops / b_kern_s / 1e12
        result["backward"] = {
            "workload": wb.name, "causal": wb.causal, "value": round(b_flops / b_step_s / 1e12, 2),
            "unit": "TFLOP/s", "ms_per_step": round(b_step_s * 1e3, 4),
            "roofline": {"kernel": "bwd_dq_kernel + bwd_dkdv_pair_kernel", "bound": "mfma",
                         "achieved": round(b_kern_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(b_kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": _sum_traffic([("bwd_dq_kernel", wb.name, BWD_SOURCES),
                                                  ("bwd_dkdv_pair_kernel", wb.name, BWD_SOURCES)])}}
    if not args.no_cpu_baseline and "prefill" in legs:
        result["cpu_baseline"] = cpu_baseline(wp, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
