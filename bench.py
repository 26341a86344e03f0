"""Benchmark of the exact attention forward on one MI355X.

One step = one attn_fwd call over the whole workload (every query row of
every head).  Default workload: causal attention, B=1, H=4, L=131072, d=64,
fp16, scale 1/8 -- the longest length of the pages' length sweep at 4 heads.
Prints ONE JSON line with throughput in TFLOP/s (algorithmic FLOPs: 4*d per
visible (query, key) pair, so causal counts only the unmasked half), the
roofline of the kernel against the dense fp16 MFMA peak, and a CPU baseline:
the fp64 oracle timed on a bounded sample of the same workload's rows (whose
GPU outputs are also checked against it).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--sweep]
    python bench.py --backward [...]

With --decode, one step is one attn_decode call (the newest Lq tokens of
each sequence of a decode workload over its paged KV cache); the metric is
bytes: the K/V rows every query row must see, read once per K/V head, plus q,
out and lse, per second, against the HBM peak.

With --compare, the kernel is timed beside standard attention (the score
matrix materialised: matmul, scale, mask, softmax, matmul, in PyTorch on the
GPU) over the pages' length sweep, with peak memory measured as the pages
do and out-of-memory recorded rather than fatal; one JSON line per length
and one summary line (speed-up and memory ratio against the pages' claims).
PyTorch's own fused attention (scaled_dot_product_attention restricted to its
FlashAttention backend) is timed beside both, as a same-machine reference.

With --backward, one step is one attn_bwd call (dq, dk, dv for an upstream
gradient, from the forward's out and lse) on the same workload, and the line
reports the backward's throughput: algorithmic FLOPs 10*d per visible pair
(the five products of the backward: scores recomputed, dP, dV, dK, dQ), i.e.
2.5 times the forward's.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import exact_io_aware_25_amd as attn  # noqa: E402
from synth import DECODE_WORKLOADS, WORKLOADS, decode_inputs, decode_lens, workload_inputs  # noqa: E402

MFMA_PEAK_F16_TFLOPS = 2516.6   # MI355X dense fp16/bf16: 256 CU x 4096 FLOP/clk x 2.4 GHz
MFMA_PEAK_F8_TFLOPS = 5033.2    # MI355X dense fp8: twice the 16-bit rate


def mfma_peak(w) -> float:
    """The dense MFMA peak of the workload's input type."""
    return MFMA_PEAK_F8_TFLOPS if w.dtype == "f8" else MFMA_PEAK_F16_TFLOPS
HBM_PEAK_GBS = 8000.0
METRIC = "causal attn fwd TFLOP/s @ L=128k,H=4,d=64 fp16; % of MFMA peak"
METRIC_BWD = "causal attn bwd TFLOP/s @ L=128k,H=4,d=64 fp16; % of MFMA peak"
METRIC_DECODE = "paged decode GB/s @ 8 x 64k-128k tokens, H=32/8, d=128 bf16; % of HBM peak"
DEFAULT_DECODE = "decode_128k_gqa"
DEFAULT_WORKLOAD = "causal_128k_h4"


def visible_pairs(L: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs the mask leaves visible in one head."""
    i = np.arange(L, dtype=np.int64)
    lo = np.zeros(L, np.int64) if window < 0 else np.maximum(0, i - window)
    if causal:
        hi = i + 1
    else:
        hi = np.full(L, L, np.int64) if window < 0 else np.minimum(L, i + window + 1)
    return int((hi - lo).sum())


def row_visible(i: np.ndarray, L: int, causal: bool, window: int) -> np.ndarray:
    lo = np.zeros_like(i) if window < 0 else np.maximum(0, i - window)
    if causal:
        hi = i + 1
    else:
        hi = np.full_like(i, L) if window < 0 else np.minimum(L, i + window + 1)
    return hi - lo


def algorithmic_flops(w) -> float:
    return 4.0 * w.d * w.B * w.H * visible_pairs(w.L, w.causal, w.window)


def algorithmic_flops_bwd(w) -> float:
    return 2.5 * algorithmic_flops(w)


def algorithmic_bytes_bwd(w) -> float:
    """One read of q, k, v, out, dout (16-bit) and lse (fp32), one write of
    dq, dk, dv (16-bit); the workspace (8 bytes per row, written and read)."""
    return (2.0 * w.B * w.L * w.d * (4 * w.H + 4 * w.H_kv) + 4.0 * w.B * w.H * w.L
            + 3 * 8.0 * w.B * w.H * w.L)


def algorithmic_bytes(w) -> float:
    """One read of q, k, v and one write of out and lse (fp32): 2 bytes per
    element for 16-bit inputs; fp8 inputs are 1 byte and their output bf16."""
    inp = 1.0 if w.dtype == "f8" else 2.0
    return (inp * w.B * w.L * w.d * (w.H + 2 * w.H_kv) + 2.0 * w.B * w.L * w.d * w.H
            + 4.0 * w.B * w.H * w.L)


def time_workload(w, steps: int, warmup: int):
    """Time `steps` calls after `warmup` calls, with HIP events recorded on the
    stream the kernel is launched on.  Peak memory is taken as the pages do:
    statistics reset after q, k, v exist, so it covers out, lse and anything
    the call itself allocates (the library allocates nothing)."""
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workload_inputs(w))
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "f8" else q.dtype, device=dev)
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        attn.forward(q, k, v, causal=w.causal, window=w.window, scale=w.scale, out=out, lse=lse,
                     stream=stream)
    torch.cuda.synchronize()
    # device memory free, by the driver's count, with the outputs allocated and
    # the code loaded: the timed calls must not change it (the library
    # allocates nothing)
    free_before = torch.cuda.mem_get_info(dev)[0]
    # one event between consecutive launches: the first and last bracket the
    # timed region (its mean is the step time), the others give each launch
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(steps):
        attn.forward(q, k, v, causal=w.causal, window=w.window, scale=w.scale, out=out, lse=lse,
                     stream=stream)
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = events[0].elapsed_time(events[-1]) / steps
    per_launch = sorted(events[i].elapsed_time(events[i + 1]) for i in range(steps))
    peak = torch.cuda.max_memory_allocated(dev)
    free_after = torch.cuda.mem_get_info(dev)[0]
    return dict(ms=ms, ms_median=per_launch[len(per_launch) // 2], ms_min=per_launch[0], wall_s=wall,
                out=out, lse=lse, inputs=(q, k, v), peak_mem=peak, peak_mem_incl_inputs=peak,
                peak_mem_call=peak - base, device_free_delta=free_before - free_after)


def input_cases(q, k, v):
    """The seeded N(0,1) inputs and three variants with the same shape and
    fewer significant bits: rounded to 8 bits (held in the input type),
    signed powers of two, zeros."""
    dt = q.dtype

    def fewer_bits(t):  # bf16 and fp8 values have 8 or fewer significant bits already
        return t.to(torch.bfloat16).to(dt) if dt == torch.float16 else t

    def pow2(t):
        f = t.float()
        return (torch.sign(f) * torch.exp2(torch.round(torch.log2(f.abs().clamp(min=2.0 ** -14))))).to(dt)

    return [("seeded N(0,1)", (q, k, v)), ("8 significant bits", tuple(fewer_bits(t) for t in (q, k, v))),
            ("signed powers of two", tuple(pow2(t) for t in (q, k, v))),
            ("zeros", tuple(torch.zeros_like(t) for t in (q, k, v)))]


def smi_sample():
    """Socket power (W), the graphics clock of every XCD (MHz) and the
    hotspot temperature (C, None if not reported) from `amd-smi metric -p -c
    -t --json`, or None where the tool or a power/clock field is missing."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-t", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    g = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else (d[0] if isinstance(d, list) else d)
    try:
        watts = float(g["power"]["socket_power"]["value"])
        clks = [float(c["clk"]["value"]) for n, c in g["clock"].items()
                if n.startswith("gfx_") and isinstance(c, dict) and isinstance(c.get("clk"), dict)]
    except (KeyError, TypeError, ValueError):
        return None
    try:
        hot = float(g["temperature"]["hotspot"]["value"])
    except (KeyError, TypeError, ValueError):
        hot = None
    return watts, clks, hot


def power_trace(w, inputs, seconds: float = 6.0):
    """Socket power, XCD clocks and hotspot temperature while the kernel runs
    back to back for about `seconds` on each input case of `input_cases` (two
    passes, so that drift over the run shows): `amd-smi` is sampled from a
    second thread once the first 2 s have passed.  One JSON line per case, to
    stderr."""
    import threading
    q, k, v = inputs
    stream = torch.cuda.current_stream()
    out = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "f8" else q.dtype, device=q.device)
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=q.device)
    for pass_no, (name, (a, b, c)) in [(p, nc) for p in (1, 2) for nc in input_cases(q, k, v)]:
        def call():
            attn.forward(a, b, c, causal=w.causal, window=w.window, scale=w.scale, out=out, lse=lse, stream=stream)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        steps = max(10, int(seconds * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
        samples, stop = [], threading.Event()

        def sampler():
            if stop.wait(2.0):
                return
            while not stop.is_set():
                smp = smi_sample()
                if smp is not None:
                    samples.append(smp)
                stop.wait(0.5)
        th = threading.Thread(target=sampler)
        th.start()
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        stop.set()
        th.join()
        ms = e0.elapsed_time(e1) / steps
        tf = algorithmic_flops(w) / (ms * 1e-3) / 1e12
        rec = {"power": name, "pass": pass_no, "workload": w.name, "steps": steps, "ms": round(ms, 4),
               "tflops": round(tf, 1), "pct_of_mfma_peak": round(100 * tf / mfma_peak(w), 2), "samples": len(samples)}
        if samples:
            rec["socket_power_w_median"] = float(np.median([s[0] for s in samples]))
            clks = [c for s in samples for c in s[1]]
            if clks:
                rec["gfx_clock_mhz_median"] = float(np.median(clks))
                rec["gfx_clock_mhz_range"] = [min(clks), max(clks)]
            hots = [s[2] for s in samples if s[2] is not None]
            if hots:
                rec["hotspot_c_max"] = max(hots)
        print(json.dumps(rec), file=sys.stderr, flush=True)


def data_sensitivity(w, inputs, steps: int):
    """The same kernel on the same shape with inputs whose values carry fewer
    significant bits: the seeded N(0,1) inputs, those values rounded to 8
    significant bits (held in the input type), signed powers of two, and
    zeros.  The instruction stream is the same in every case (the sum-checked
    softmax takes its slow path only on each row block's first tile either
    way), so a change of time is a change of clock: the MFMA arrays draw less
    power on operands with fewer bits set.  One JSON line per case, to stderr."""
    q, k, v = inputs
    dt = q.dtype
    cases = input_cases(q, k, v)
    stream = torch.cuda.current_stream()
    out = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "f8" else dt, device=q.device)
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=q.device)
    # two passes over the cases, so that a drift of the clock over the run
    # (it differs from the first case to the last) shows as a difference
    # between the passes rather than between the cases
    for pass_no, (name, (a, b, c)) in [(p, nc) for p in (1, 2) for nc in cases]:
        for _ in range(3):
            attn.forward(a, b, c, causal=w.causal, window=w.window, scale=w.scale, out=out, lse=lse, stream=stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            attn.forward(a, b, c, causal=w.causal, window=w.window, scale=w.scale, out=out, lse=lse, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = algorithmic_flops(w) / (ms * 1e-3) / 1e12
        print(json.dumps({"data_sensitivity": name, "pass": pass_no, "workload": w.name, "ms": round(ms, 4),
                          "tflops": round(tf, 1), "pct_of_mfma_peak": round(100 * tf / mfma_peak(w), 2)}),
              file=sys.stderr, flush=True)


def decode_bytes(w) -> float:
    """Algorithmic bytes of one decode step: every K/V row some query row
    sees, once per K/V head, plus q and out (16-bit), lse (fp32), the page
    table entries and lengths."""
    kv = 0
    for n in decode_lens(w):
        first = max(0, n - w.Lq - w.window) if w.window >= 0 else 0
        kv += (n - first) * w.H_kv * w.d * 2 * 2
        kv += 4 * ((n + w.block_size - 1) // w.block_size) + 4
    rows = w.B * w.H * w.Lq
    return float(kv + rows * w.d * 2 * 2 + rows * 4)


def time_decode(w, steps: int, warmup: int):
    dev = torch.device("cuda:0")
    q, kc, vc, bt, sl = (t.to(dev) for t in decode_inputs(w))
    max_len = max(decode_lens(w))
    stream = torch.cuda.current_stream(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.empty(attn.attn_decode_workspace_size(w.B, w.H, w.H_kv, w.Lq, w.d, max_len), dtype=torch.uint8,
                     device=dev)

    def step():
        attn.decode(q, kc, vc, bt, sl, max_len, window=w.window, scale=w.scale, out=out, lse=lse,
                    workspace=ws, stream=stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    return dict(ms=start.elapsed_time(stop) / steps, out=out, lse=lse, workspace_bytes=ws.numel(),
                inputs=(q, kc, vc, bt, sl))


def cpu_baseline_decode(w, out, inputs, budget_s: float = 15.0):
    """The fp64 paged oracle (NumPy, BLAS threads up to the host cores) on
    whole sequences, in order, for about `budget_s` seconds; its throughput in
    the metric's bytes, and the GPU's error on those sequences."""
    from threadpoolctl import threadpool_limits

    from oracle import paged
    q, kc, vc, bt, sl = (t.cpu() for t in inputs)
    lens = decode_lens(w)
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    done, nbytes, elapsed, err = 0, 0.0, 0.0, 0.0
    with threadpool_limits(limits=threads):
        while done < w.B and elapsed < budget_s:
            b = done
            t0 = time.perf_counter()
            ro, _ = paged.decode_attention(q[b:b + 1], kc, vc, bt[b:b + 1].numpy(), [lens[b]], w.dtype,
                                           w.window, w.scale)
            elapsed += time.perf_counter() - t0
            n = lens[b]
            first = max(0, n - w.Lq - w.window) if w.window >= 0 else 0
            nbytes += (n - first) * w.H_kv * w.d * 4 + w.H * w.Lq * (w.d * 4 + 4)
            err = max(err, float(np.abs(out[b:b + 1].double().cpu().numpy() - ro).max()))
            done += 1
    return dict(value=nbytes / elapsed / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{done} of {w.B} sequences of {w.name}, {elapsed:.1f} s of fp64 oracle time",
                parity_max_abs_o=err)


def make_dout(w):
    """The upstream gradient of the backward benchmark: seeded N(0,1), rounded."""
    from synth import make_qkv
    g, _, _ = make_qkv(w.B, w.H, w.H, w.L, w.d, w.dtype, 5007)
    return g


def time_backward(w, steps: int, warmup: int):
    """Forward once, then time `steps` backward calls after `warmup` calls,
    with HIP events on the stream the kernels are launched on."""
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workload_inputs(w))
    g = make_dout(w).to(dev)
    stream = torch.cuda.current_stream(dev)
    out, lse = attn.forward(q, k, v, causal=w.causal, window=w.window, scale=w.scale, stream=stream)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(attn.attn_bwd_workspace_size(w.B, w.H, w.L), dtype=torch.uint8, device=dev)

    def step():
        attn.backward(q, k, v, out, lse, g, causal=w.causal, window=w.window, scale=w.scale,
                      dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / steps
    peak = torch.cuda.max_memory_allocated(dev)
    return dict(ms=ms, wall_s=wall, dq=dq, inputs=(q, k, v, g), peak_mem_call=peak - base)


def cpu_baseline_bwd(w, dq, inputs, budget_s: float = 15.0, seed: int = 7):
    """Time the fp64 backward oracle computing dq for a seeded sample of query
    rows for about `budget_s` seconds.  Its work is counted as 6*d FLOPs per
    visible pair of those rows (scores, dP and dq: what it computes for them);
    the GPU's dq on those rows is compared with it."""
    import oracle
    q, k, v, g = (t.cpu() for t in inputs)
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    rng = np.random.default_rng(seed)
    n_total = w.B * w.H * w.L
    order = rng.permutation(n_total)
    done, flops, elapsed, err = 0, 0.0, 0.0, 0.0
    flat = dq.reshape(-1, w.d)
    batch = 32
    while elapsed < budget_s and done < n_total:
        rows = np.sort(order[done:done + batch])
        t0 = time.perf_counter()
        ref, _, _ = oracle.attention_bwd(q, k, v, g, w.dtype, w.causal, w.window, w.scale,
                                         q_rows=rows, kv_rows=[], threads=threads)
        elapsed += time.perf_counter() - t0
        flops += 6.0 * w.d * float(row_visible(rows % w.L, w.L, w.causal, w.window).sum())
        got = flat[torch.from_numpy(rows).to(flat.device)].double().cpu().numpy()
        err = max(err, float(np.abs(got - ref).max()))
        done += len(rows)
        batch = min(2048, batch * 2)
    return dict(value=flops / elapsed / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"dq of {done} seeded random query rows of {n_total} ({w.name}), "
                       f"{elapsed:.1f} s of fp64 oracle time, {flops:.3e} FLOPs (6*d per visible pair)",
                parity_max_abs_dq=err)


def cpu_baseline(w, out, lse, inputs, budget_s: float = 15.0, seed: int = 7):
    """Time the fp64 oracle on a seeded sample of rows for about `budget_s`
    seconds; return its throughput in the metric's unit and the GPU-vs-oracle
    error on those rows."""
    import oracle
    q, k, v = (t.cpu() for t in inputs)
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    rng = np.random.default_rng(seed)
    n_total = w.B * w.H * w.L
    order = rng.permutation(n_total)
    done, flops, elapsed = 0, 0.0, 0.0
    err_o, err_l = 0.0, 0.0
    flat_o = out.reshape(-1, w.d)
    flat_l = lse.reshape(-1)
    batch = 64
    while elapsed < budget_s and done < n_total:
        rows = np.sort(order[done:done + batch])
        t0 = time.perf_counter()
        ro, rl = oracle.attention(q, k, v, w.dtype, w.causal, w.window, w.scale, rows=rows, threads=threads)
        elapsed += time.perf_counter() - t0
        flops += 4.0 * w.d * float(row_visible(rows % w.L, w.L, w.causal, w.window).sum())
        idx = torch.from_numpy(rows)
        go = flat_o[idx.to(flat_o.device)].double().cpu().numpy()
        gl = flat_l[idx.to(flat_l.device)].double().cpu().numpy()
        err_o = max(err_o, float(np.abs(go - ro).max()))
        err_l = max(err_l, float(np.abs(gl - rl).max()))
        done += len(rows)
        batch = min(4096, batch * 2)
    rate = flops / elapsed
    return dict(value=rate / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{done} seeded random query rows of {n_total} ({w.name}), "
                       f"{elapsed:.1f} s of fp64 oracle time, {flops:.3e} algorithmic FLOPs",
                extrapolated_full_s=round(algorithmic_flops(w) / rate, 1), cpu_model=cpu_model(),
                parity_max_abs_o=err_o, parity_max_abs_lse=err_l)


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_io_aware_25_amd", "csrc")
KERNEL_SOURCE = os.path.join(CSRC, "attn_fwd.hip")
KERNEL_SOURCE_BWD = os.path.join(CSRC, "attn_bwd.hip")
KERNEL_SOURCE_DECODE = os.path.join(CSRC, "attn_decode.hip")
KERNEL_SOURCE_F8 = os.path.join(CSRC, "attn_fwd_f8.hip")


def kernel_source_sha256(path: str = KERNEL_SOURCE) -> str:
    """Hash of a kernel source followed by the shared header it includes."""
    import hashlib
    h = hashlib.sha256(open(path, "rb").read())
    h.update(open(os.path.join(CSRC, "attn_common.h"), "rb").read())
    return h.hexdigest()


def profiled_traffic(w, kind: str = "attn_fwd", source: str = KERNEL_SOURCE):
    """Bytes per launch between L2 and memory for this workload, from the
    committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE per
    dispatch, each scaled by what the counter reads for a plain device copy
    of known size); None when there is no summary for this workload or the
    kernel source has changed since it was taken."""
    path = os.path.join(PROFILES, f"{kind}_{w.name}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            vals[key.strip()] = val.strip()
    if vals.get("workload") != w.name or vals.get("kernel_source_sha256") != kernel_source_sha256(source):
        return None
    copy_bytes = float(vals["copy_bytes"])
    fetch_scale = copy_bytes / (float(vals["copy_fetch_kib"]) * 1024)
    write_scale = copy_bytes / (float(vals["copy_write_kib"]) * 1024)
    return (float(vals["fetch_kib_per_dispatch"]) * 1024 * fetch_scale
            + float(vals["write_kib_per_dispatch"]) * 1024 * write_scale)


def profiled_request_traffic(w, kind: str = "attn_fwd", source: str = KERNEL_SOURCE):
    """Bytes per launch between L2 and memory counted from the request-size
    counters (TCC_EA0_RDREQ_32B/64B/128B and TCC_EA0_WRREQ/WRREQ_64B, each
    request times its size), scaled by what the same counters read for a plain
    device copy of known size; None when there is no summary for this workload
    or the kernel source has changed since it was taken.  FETCH_SIZE estimates
    128-byte reads from a bubble counter, and on gfx950 its ratio to the true
    bytes differs between kernels with the same request sizes, so its copy
    scaling is not exact; the request counts are."""
    path = os.path.join(PROFILES, f"{kind}_{w.name}_requests.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            vals[key.strip()] = val.strip()
    if vals.get("workload") != w.name or vals.get("kernel_source_sha256") != kernel_source_sha256(source):
        return None
    copy_bytes = float(vals["copy_bytes"])
    read_scale = copy_bytes / float(vals["copy_read_bytes"])
    write_scale = copy_bytes / float(vals["copy_write_bytes"])
    return (float(vals["read_bytes_per_launch"]) * read_scale
            + float(vals["write_bytes_per_launch"]) * write_scale)


def roofline_block(w, ms):
    flops = algorithmic_flops(w)
    achieved = flops / (ms * 1e-3) / 1e12
    peak = mfma_peak(w)
    source = KERNEL_SOURCE_F8 if w.dtype == "f8" else KERNEL_SOURCE
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": profiled_traffic(w, "attn_fwd", source),
            "traffic_requests": profiled_request_traffic(w, "attn_fwd", source)}


ORACLE_TIMING_WORKLOADS = ("p2_accuracy", "causal_4k", "noncausal_2k_f16", "noncausal_2k_bf16", "causal_8k",
                           "causal_16k", "causal_32k", "swa_gqa_16k")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_timings(steps: int):
    """The whole fp64 oracle (every row) on the host cores for the workloads
    whose oracle finishes in seconds to a minute, beside the GPU's median and
    minimum launch time of the same workload and the parity of every output
    element; one JSON line per workload, to stderr."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    model = cpu_model()
    for name in ORACLE_TIMING_WORKLOADS:
        w = WORKLOADS[name]
        r = time_workload(w, steps, 5)
        q, k, v = (t.cpu() for t in r["inputs"])
        t0 = time.perf_counter()
        ref_o, ref_l = oracle.attention(q, k, v, w.dtype, w.causal, w.window, w.scale, threads=threads)
        cpu_s = time.perf_counter() - t0
        err_o = np.abs(r["out"].double().cpu().numpy() - ref_o)
        err_l = np.abs(r["lse"].double().cpu().numpy() - ref_l)
        flops = algorithmic_flops(w)
        print(json.dumps({"oracle_timing": name, "dtype": w.dtype, "B": w.B, "H": w.H, "H_kv": w.H_kv, "L": w.L,
                          "d": w.d, "causal": w.causal, "window": w.window,
                          "oracle_s": round(cpu_s, 3), "oracle_tflops": flops / cpu_s / 1e12,
                          "cores": threads, "cpu_model": model,
                          "gpu_ms_mean": round(r["ms"], 5), "gpu_ms_median": round(r["ms_median"], 5),
                          "gpu_ms_min": round(r["ms_min"], 5), "gpu_over_oracle": round(cpu_s / (r["ms"] * 1e-3), 1),
                          "max_abs_o": float(err_o.max()), "mean_abs_o": float(err_o.mean()),
                          "max_abs_lse": float(err_l.max())}), file=sys.stderr, flush=True)
        del r
        torch.cuda.empty_cache()


def write_csv(path, header, rows):
    """The results file of the pages' benchmark assignment: one row per
    length with time and peak memory, "OOM" where a run ran out of memory."""
    import csv
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)
    print(f"bench.py: wrote {len(rows)} rows to {path}", file=sys.stderr, flush=True)


def loglog_slope(xs, ys):
    lx, ly = np.log(np.asarray(xs, float)), np.log(np.asarray(ys, float))
    return float(np.polyfit(lx, ly, 1)[0])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS) + sorted(DECODE_WORKLOADS))
    ap.add_argument("--sweep", action="store_true",
                    help="also time every workload and print one extra JSON line each (to stderr); with "
                         "--backward every 16-bit workload's backward, with --decode every decode workload")
    ap.add_argument("--data-sensitivity", action="store_true",
                    help="also time the workload's kernel on inputs with fewer significant bits (same "
                         "shape, same instructions) and print one extra JSON line each (to stderr); "
                         "with --backward: N(0,1) and zero inputs")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="time the paged decode (attn_decode) on a decode workload")
    ap.add_argument("--compare", action="store_true",
                    help="time the kernel beside standard attention over the pages' length sweep")
    ap.add_argument("--oracle-timings", action="store_true",
                    help="also run the whole fp64 oracle on the host cores for the workloads it finishes in about a "
                         "minute or less (one JSON line each, to stderr, with the GPU's median and minimum times)")
    ap.add_argument("--csv", default=None,
                    help="with --sweep or --compare, also write the per-length results (L, time_ms, mem_GB, "
                         "'OOM' where standard attention ran out of memory) to this CSV file")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (attn_bwd) on the workload instead of the forward")
    ap.add_argument("--power", action="store_true",
                    help="also run the forward for ~6 s on each input case of --data-sensitivity while sampling "
                         "socket power, XCD clocks and hotspot temperature with amd-smi; one JSON line per case "
                         "(to stderr)")
    ap.add_argument("--torch-flash", action="store_true",
                    help="also time PyTorch's fused attention (FlashAttention backend) on the same inputs, "
                         "forward or backward; one JSON line to stderr")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a reference "
                         "kernel of known traffic for scaling profiler byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library and this benchmark run on one GPU; --gpus {args.gpus} is not supported "
              "(the kernel shards over (batch, head) with no exchange, so N GPUs run N independent "
              "copies).", file=sys.stderr)
        sys.exit(2)

    attn.library()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.float16, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.compare:
        main_compare(args)
        return
    if args.decode or args.workload in DECODE_WORKLOADS:
        main_decode(DECODE_WORKLOADS[args.workload or DEFAULT_DECODE], args)
        return
    w = WORKLOADS[args.workload or DEFAULT_WORKLOAD]
    if args.backward:
        main_backward(w, args)
        return
    r = time_workload(w, args.steps, args.warmup)
    flops = algorithmic_flops(w)
    tflops = flops / (r["ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC if w.name == DEFAULT_WORKLOAD else f"attn fwd TFLOP/s ({w.name})",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded iid N(0,1) q, k, v rounded to the input type",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "L": w.L, "d": w.d,
                   "causal": w.causal, "window": w.window, "scale": w.scale,
                   "algorithmic_flops": flops, "pct_of_mfma_peak": round(100 * tflops / mfma_peak(w), 2),
                   "ms_median": round(r["ms_median"], 4), "ms_min": round(r["ms_min"], 4),
                   "peak_mem_bytes": r["peak_mem"], "peak_mem_call_bytes": r["peak_mem_call"],
                   "device_free_delta_bytes": r["device_free_delta"],
                   "algorithmic_bytes": algorithmic_bytes(w)},
        "roofline": roofline_block(w, r["ms"]),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, r["out"], r["lse"], r["inputs"], args.cpu_budget)
    print(json.dumps(line), flush=True)

    if args.data_sensitivity:
        data_sensitivity(w, r["inputs"], max(5, args.steps))
    if args.torch_flash and w.dtype in ("f16", "bf16"):
        torch_flash(w, r["inputs"], args.steps, args.warmup, False, r["ms"])
    if args.power:
        power_trace(w, r["inputs"])

    r = line = None  # the headline's tensors are no longer needed
    torch.cuda.empty_cache()
    if args.oracle_timings:
        oracle_timings(max(10, args.steps))

    if args.sweep:
        sweep = []
        for name, ws in WORKLOADS.items():
            # 10 warm-up and 100 timed calls up to 32k tokens, 3 and 20 beyond
            # (or --steps, if larger)
            short = ws.L <= 32768
            steps, warm = max(100 if short else 20, args.steps), 10 if short else 3
            try:
                rs = time_workload(ws, steps, warm)
            except torch.cuda.OutOfMemoryError:
                rec = {"workload": name, "dtype": ws.dtype, "L": ws.L, "ms": "OOM", "ms_median": "OOM",
                       "ms_min": "OOM", "tflops": "OOM", "pct_peak": "OOM", "peak_mem_bytes": "OOM"}
                sweep.append(rec)
                print(json.dumps(rec), file=sys.stderr, flush=True)
                torch.cuda.empty_cache()
                continue
            f = algorithmic_flops(ws)
            rec = {"workload": name, "dtype": ws.dtype, "L": ws.L, "steps": steps, "warmup": warm,
                   "ms": round(rs["ms"], 4), "ms_median": round(rs["ms_median"], 4), "ms_min": round(rs["ms_min"], 4),
                   "tflops": round(f / (rs["ms"] * 1e-3) / 1e12, 2),
                   "pct_peak": round(100 * f / (rs["ms"] * 1e-3) / 1e12 / mfma_peak(ws), 2),
                   "peak_mem_bytes": rs["peak_mem"], "peak_mem_call_bytes": rs["peak_mem_call"],
                   "algorithmic_bytes": algorithmic_bytes(ws)}
            sweep.append(rec)
            print(json.dumps(rec), file=sys.stderr, flush=True)
            del rs
            torch.cuda.empty_cache()
        # the pages' length sweep (causal, B=1, H=4, d=64): log-log slopes of time and memory
        pts = sorted((rec["L"], rec["ms"], rec["peak_mem_bytes"]) for rec in sweep
                     if rec["workload"] in ("causal_4k", "causal_8k", "causal_16k", "causal_32k",
                                            "causal_64k", "causal_128k_h4") and rec["ms"] != "OOM")
        Ls, ts, ms_ = zip(*pts)
        print(json.dumps({"length_sweep": {"L": Ls, "ms": ts, "peak_mem_bytes": ms_,
                                           "slope_time": round(loglog_slope(Ls, ts), 3),
                                           "slope_memory": round(loglog_slope(Ls, ms_), 3)}}),
              file=sys.stderr, flush=True)
        if args.csv:
            write_csv(args.csv, ["workload", "dtype", "L", "time_ms", "time_ms_median", "time_ms_min", "mem_GB",
                                 "tflops", "pct_peak"],
                      [[r["workload"], r["dtype"], r["L"], r["ms"], r["ms_median"], r["ms_min"],
                        "OOM" if r["peak_mem_bytes"] == "OOM" else round(r["peak_mem_bytes"] / 1e9, 6),
                        r["tflops"], r["pct_peak"]] for r in sweep])


def standard_attention(q, k, v, causal: bool, scale: float, rows_per_step: int = 8192,
                       split_above: int = 1 << 31):
    """Attention with the score matrix materialised (the pages' 'standard
    attention': matmul, softmax, matmul), 16-bit like the inputs; a
    comparator only, never part of the library.  Up to 2^31 score elements it
    is the plain three-step version; above, the whole [B,H,L,L] score and
    weight matrices still exist at once, but every operation works on one
    (batch, head) and a block of query rows, so that none indexes more than
    ~2^30 elements (single products over larger tensors gave wrong results
    at 64k here)."""
    B, H, L, d = q.shape
    kt = k.transpose(-1, -2).contiguous()
    if B * H * L * L < split_above:
        # small enough for single operations: the plain three-step version
        s = torch.matmul(q, kt)
        del kt
        s.mul_(scale)
        if causal:
            s.masked_fill_(torch.ones(L, L, dtype=torch.bool, device=q.device).triu_(1), float("-inf"))
        p = torch.softmax(s, dim=-1)
        del s
        return torch.matmul(p, v)
    s = torch.empty((B, H, L, L), dtype=q.dtype, device=q.device)
    p = torch.empty_like(s)
    out = torch.empty_like(q)
    step = max(1, min(L, (1 << 30) // max(1, L), rows_per_step))
    cols = torch.arange(L, device=q.device)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, L, step):
                r1 = min(L, r0 + step)
                blk = s[b, h, r0:r1]
                torch.matmul(q[b, h, r0:r1], kt[b, h], out=blk)
                blk.mul_(scale)
                if causal:
                    blk.masked_fill_(cols[None, :] > torch.arange(r0, r1, device=q.device)[:, None], float("-inf"))
                p[b, h, r0:r1] = torch.softmax(blk, dim=-1)
    del s
    for b in range(B):
        for h in range(H):
            for r0 in range(0, L, step):
                r1 = min(L, r0 + step)
                torch.matmul(p[b, h, r0:r1], v[b, h], out=out[b, h, r0:r1])
    return out


def compare_one(B, H, L, d, causal, scale, seed, reps=3):
    """Time and peak memory of the kernel and of standard attention at one
    shape (statistics reset after q, k, v exist, as the pages measure)."""
    from synth import make_qkv
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_qkv(B, H, H, L, d, "f16", seed))
    res = {"B": B, "H": H, "L": L, "d": d, "causal": causal}

    def measure(fn):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        out = fn()  # warm-up call, also the one whose memory peak is kept
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        times = []
        for _ in range(reps):
            del out
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            out = fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2], peak, out

    t_f, m_f, o_f = measure(lambda: attn.forward(q, k, v, causal=causal, scale=scale)[0])
    res.update(flash_ms=round(t_f, 4), flash_peak_bytes=m_f)
    # PyTorch's own fused attention (its FlashAttention backend, precompiled
    # for this GPU), timed the same way: a same-machine point of comparison
    # for the kernel, not part of the pages' claims.
    from torch.nn.attention import SDPBackend, sdpa_kernel
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            t_l, m_l, o_l = measure(lambda: torch.nn.functional.scaled_dot_product_attention(
                q, k, v, is_causal=causal, scale=scale))
        res.update(torch_flash_ms=round(t_l, 4), torch_flash_peak_bytes=m_l,
                   torch_flash_max_abs_diff=float((o_l.float() - o_f.float()).abs().max()),
                   kernel_over_torch_flash=round(t_l / t_f, 2))
        del o_l
    except RuntimeError as e:  # backend not built for this GPU or shape
        res.update(torch_flash_ms=None, torch_flash_error=str(e).splitlines()[0][:200])
    try:
        t_s, m_s, o_s = measure(lambda: standard_attention(q, k, v, causal, scale))
        diff = float((o_s.float() - o_f.float()).abs().max())
        res.update(standard_ms=round(t_s, 4), standard_peak_bytes=m_s, speedup=round(t_s / t_f, 2),
                   memory_ratio=round(m_s / m_f, 1), max_abs_diff=diff,
                   # fp16 scores and weights put the comparator itself ~1e-3 off
                   standard_result_valid=diff < 1e-2)
        del o_s
    except torch.cuda.OutOfMemoryError:
        res.update(standard_ms=None, standard_peak_bytes="OOM")
    del o_f, q, k, v
    torch.cuda.empty_cache()
    return res


def torch_flash(w, inputs, steps: int, warmup: int, backward: bool, ms_kernel: float):
    """PyTorch's own fused attention on the same inputs: scaled_dot_product_attention
    restricted to its FlashAttention backend (precompiled for this GPU), the
    forward call, or the backward alone (autograd over a retained forward
    graph), timed with HIP events like the kernel.  A same-machine point of
    comparison only; one JSON line to stderr.  Windows have no counterpart
    there, and a grouped K/V layout is passed as enable_gqa."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    rec = {"torch_flash": w.name, "pass": "backward" if backward else "forward", "torch": torch.__version__}
    if w.window >= 0:
        rec["error"] = "no sliding-window form in scaled_dot_product_attention"
        print(json.dumps(rec), file=sys.stderr, flush=True)
        return rec
    q, k, v = (t.detach().requires_grad_(backward) for t in inputs[:3])
    kw = dict(is_causal=w.causal, scale=w.scale, enable_gqa=w.H_kv != w.H)
    steps = max(1, steps)
    res = None
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            if backward:
                out = torch.nn.functional.scaled_dot_product_attention(q, k, v, **kw)
                g = inputs[3]

                def step():
                    return torch.autograd.grad(out, (q, k, v), g, retain_graph=True)
            else:
                def step():
                    return torch.nn.functional.scaled_dot_product_attention(q, k, v, **kw)
            for _ in range(warmup):
                res = step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                res = step()
            e1.record()
            torch.cuda.synchronize()
    except RuntimeError as e:  # backend not built for this GPU, shape or dtype
        rec["error"] = str(e).splitlines()[0][:200]
        print(json.dumps(rec), file=sys.stderr, flush=True)
        return rec
    ms = e0.elapsed_time(e1) / steps
    flops = algorithmic_flops_bwd(w) if backward else algorithmic_flops(w)
    tf = flops / (ms * 1e-3) / 1e12
    rec.update(ms=round(ms, 4), tflops=round(tf, 1), pct_of_mfma_peak=round(100 * tf / MFMA_PEAK_F16_TFLOPS, 2),
               kernel_speedup=round(ms / ms_kernel, 2))
    del res
    print(json.dumps(rec), file=sys.stderr, flush=True)
    return rec


def main_compare(args):
    """The pages' sweep (causal, B=1, H=4, d=64, fp16, 512 ... 128k) and the
    speed-check shape (B=2, H=8, L=2048, d=64, no mask)."""
    rows = []
    shapes = [(1, 4, L, 64, True) for L in (512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)]
    shapes.append((2, 8, 2048, 64, False))
    for i, (B, H, L, d, causal) in enumerate(shapes):
        r = compare_one(B, H, L, d, causal, 0.125, 3000 + i)
        rows.append(r)
        print(json.dumps({"compare": r}), flush=True)
    if args.csv:
        def std(r, key, scale=1.0):
            v = r.get(key)
            return "OOM" if r.get("standard_peak_bytes") == "OOM" else (round(v / scale, 6) if v is not None else "")
        write_csv(args.csv, ["B", "H", "L", "d", "causal", "time_ms", "mem_GB", "standard_time_ms",
                             "standard_mem_GB", "speedup", "memory_ratio", "torch_flash_time_ms"],
                  [[r["B"], r["H"], r["L"], r["d"], int(r["causal"]), r["flash_ms"],
                    round(r["flash_peak_bytes"] / 1e9, 6), std(r, "standard_ms"),
                    std(r, "standard_peak_bytes", 1e9), r.get("speedup", ""), r.get("memory_ratio", ""),
                    r.get("torch_flash_ms") or ""]
                   for r in rows])
    ok = [r for r in rows if r.get("standard_ms") and r.get("standard_result_valid")]
    lib = [r for r in rows if r.get("torch_flash_ms")]
    print(json.dumps({"compare_summary": {
        "speedup_range": [min(r["speedup"] for r in ok), max(r["speedup"] for r in ok)],
        "memory_ratio_range": [min(r["memory_ratio"] for r in ok), max(r["memory_ratio"] for r in ok)],
        "standard_oom_at": [r["L"] for r in rows if r.get("standard_peak_bytes") == "OOM"],
        "kernel_over_torch_flash_range": [min(r["kernel_over_torch_flash"] for r in lib),
                                          max(r["kernel_over_torch_flash"] for r in lib)] if lib else None,
        "claims": "2-4x faster (more at longer sequences), 10-20x less memory, standard attention OOM at 128k",
    }}), flush=True)


def main_decode(w, args):
    r = time_decode(w, args.steps, args.warmup)
    nbytes = decode_bytes(w)
    gbs = nbytes / (r["ms"] * 1e-3) / 1e9
    lens = decode_lens(w)
    line = {
        "metric": METRIC_DECODE if w.name == DEFAULT_DECODE else f"paged decode GB/s ({w.name})",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded iid N(0,1) q and KV cache rounded to the 16-bit type; seeded ragged "
                "lengths and shuffled block tables",
        "config": {"workload": w.name, "pass": "decode", "B": w.B, "H": w.H, "H_kv": w.H_kv, "d": w.d,
                   "Lq": w.Lq, "block_size": w.block_size, "window": w.window, "scale": w.scale,
                   "seq_len_min": min(lens), "seq_len_max": max(lens), "algorithmic_bytes": nbytes,
                   "workspace_bytes": r["workspace_bytes"], "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                   "launches_per_step": 2},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(w, "attn_decode", KERNEL_SOURCE_DECODE),
                     "traffic_requests": profiled_request_traffic(w, "attn_decode", KERNEL_SOURCE_DECODE),
                     "scope": "one attn_decode call (partial and merge kernels)"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(w, r["out"], r["inputs"], args.cpu_budget)
    print(json.dumps(line), flush=True)
    if args.sweep:
        r = line = None
        torch.cuda.empty_cache()
        rows = []
        for name, wd in DECODE_WORKLOADS.items():
            rs = time_decode(wd, max(100, args.steps), 10)
            nb = decode_bytes(wd)
            rec = {"decode_sweep": name, "dtype": wd.dtype, "B": wd.B, "Lq": wd.Lq, "steps": max(100, args.steps),
                   "ms": round(rs["ms"], 4), "gbs": round(nb / (rs["ms"] * 1e-3) / 1e9, 1),
                   "pct_hbm_peak": round(100 * nb / (rs["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                   "algorithmic_bytes": nb}
            rows.append(rec)
            print(json.dumps(rec), file=sys.stderr, flush=True)
            del rs
            torch.cuda.empty_cache()
        if args.csv:
            write_csv(args.csv, ["workload", "dtype", "B", "Lq", "time_ms", "GB_per_s", "pct_hbm_peak", "bytes"],
                      [[r_["decode_sweep"], r_["dtype"], r_["B"], r_["Lq"], r_["ms"], r_["gbs"], r_["pct_hbm_peak"],
                        r_["algorithmic_bytes"]] for r_ in rows])


def bwd_launches(w) -> int:
    """Kernel launches of one attn_bwd call: prep, then dK/dV and dQ, which
    share one launch at d=64 when both together have at most 9 workgroups
    (128 rows each) per CU."""
    n_blk = (w.L + 127) // 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 2 if w.d == 64 and n_blk * w.B * (w.H_kv + w.H) <= 9 * cus else 3


def main_backward(w, args):
    r = time_backward(w, args.steps, args.warmup)
    flops = algorithmic_flops_bwd(w)
    tflops = flops / (r["ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC_BWD if w.name == DEFAULT_WORKLOAD else f"attn bwd TFLOP/s ({w.name})",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded iid N(0,1) q, k, v and upstream gradient, rounded to the 16-bit type",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "H": w.H, "H_kv": w.H_kv, "L": w.L,
                   "d": w.d, "causal": w.causal, "window": w.window, "scale": w.scale,
                   "algorithmic_flops": flops, "pct_of_mfma_peak": round(100 * tflops / MFMA_PEAK_F16_TFLOPS, 2),
                   "peak_mem_call_bytes": r["peak_mem_call"], "algorithmic_bytes": algorithmic_bytes_bwd(w),
                   "launches_per_step": bwd_launches(w)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_F16_TFLOPS, 4),
                     "traffic": profiled_traffic(w, "attn_bwd", KERNEL_SOURCE_BWD),
                     "traffic_requests": profiled_request_traffic(w, "attn_bwd", KERNEL_SOURCE_BWD),
                     "scope": "one attn_bwd call (prep, then dK/dV and dQ: one launch each, or one shared "
                              "launch on short d=64 grids)"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(w, r["dq"], r["inputs"], args.cpu_budget)
    print(json.dumps(line), flush=True)
    if args.data_sensitivity:
        data_sensitivity_bwd(w, r["inputs"], max(3, args.steps // 4))
    if args.torch_flash:
        torch_flash(w, r["inputs"], args.steps, args.warmup, True, r["ms"])
    if args.sweep:
        r = line = None
        torch.cuda.empty_cache()
        rows = []
        for name, ws in WORKLOADS.items():
            if ws.dtype == "f8":
                continue  # the backward takes 16-bit inputs
            short = ws.L <= 32768
            steps, warm = max(50 if short else 10, args.steps), 5 if short else 2
            rs = time_backward(ws, steps, warm)
            f = algorithmic_flops_bwd(ws)
            rec = {"backward_sweep": name, "dtype": ws.dtype, "L": ws.L, "steps": steps, "warmup": warm,
                   "ms": round(rs["ms"], 4), "tflops": round(f / (rs["ms"] * 1e-3) / 1e12, 2),
                   "pct_peak": round(100 * f / (rs["ms"] * 1e-3) / 1e12 / MFMA_PEAK_F16_TFLOPS, 2),
                   "peak_mem_call_bytes": rs["peak_mem_call"]}
            rows.append(rec)
            print(json.dumps(rec), file=sys.stderr, flush=True)
            del rs
            torch.cuda.empty_cache()
        if args.csv:
            write_csv(args.csv, ["workload", "dtype", "L", "time_ms", "tflops", "pct_peak", "mem_GB"],
                      [[r_["backward_sweep"], r_["dtype"], r_["L"], r_["ms"], r_["tflops"], r_["pct_peak"],
                        round(r_["peak_mem_call_bytes"] / 1e9, 6)] for r_ in rows])


def data_sensitivity_bwd(w, inputs, steps: int):
    """The backward pass on the seeded N(0,1) inputs and on zeros (same
    instruction stream), two passes; one JSON line per case, to stderr.  As for
    the forward, a change of time is a change of clock."""
    q, k, v, g = inputs
    stream = torch.cuda.current_stream()
    ws = torch.empty(attn.attn_bwd_workspace_size(w.B, w.H, w.L), dtype=torch.uint8, device=q.device)
    cases = [("seeded N(0,1)", (q, k, v, g)), ("zeros", tuple(torch.zeros_like(t) for t in (q, k, v, g)))]
    for pass_no, (name, (a, b, c, d)) in [(p, nc) for p in (1, 2) for nc in cases]:
        out, lse = attn.forward(a, b, c, causal=w.causal, window=w.window, scale=w.scale, stream=stream)
        dq, dk, dv = torch.empty_like(a), torch.empty_like(b), torch.empty_like(c)

        def step():
            attn.backward(a, b, c, out, lse, d, causal=w.causal, window=w.window, scale=w.scale,
                          dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = algorithmic_flops_bwd(w) / (ms * 1e-3) / 1e12
        print(json.dumps({"data_sensitivity": name, "pass": pass_no, "workload": w.name, "backward": True,
                          "ms": round(ms, 4), "tflops": round(tf, 1),
                          "pct_of_mfma_peak": round(100 * tf / MFMA_PEAK_F16_TFLOPS, 2)}),
              file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
