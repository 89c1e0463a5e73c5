#!/usr/bin/env python3
"""Throughput of the linear-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one causal forward (linattn_forward, bf16 storage, fp32 state)
over the long-context workload B=2, H=8, N=131072, C=M=64: the chunk
kernels, the segment scan and the causal walk.  `value` is whole-job
tokens/s (B*N sequence positions per second, every head included) with the
inputs resident in HBM.  The same run also times
  * the same forward as single cold calls (a 512 MB read between calls
    evicts the caches), and a plain device copy for the measured ceiling,
  * the recurrent decode step on 256 sequences x 8 heads for 3072 steps
    (captured in one HIP graph, one kernel per step), and on 8x the heads,
  * the causal forward on B=16, H=8, N=3072 and the non-causal forward on
    B=8, H=8, N=4096, warm and cold, and the fp32 B=1, H=1, N=256 forward
    (host-inclusive, device-only from a HIP graph replay, and cold),
  * the backward (dQ, dK, dV) of the headline and CIFAR-shaped workloads,
  * forward and forward+backward time and peak memory for N = 2^9..2^16,
  * images/s of greedy generation with a random-weight 12-layer shell
    (3072 steps for 256 images, attention through the decode step),
  * the fp64 CPU oracle on a bounded sample of the headline workload
    (`cpu_baseline`, rank 0 only).
`roofline` is for the dominant kernel (the causal walk): algorithmic bytes
per launch over its average duration from HIP events recorded on the launch
stream during the timed steps; `roofline.whole_call` puts the same bytes over
the whole call.  `traffic` comes from the committed
rocprofv3 FETCH_SIZE / WRITE_SIZE summary when it was taken on the current
kernel sources, else null.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal linear-attn fwd tokens/s + % HBM/MFMA roofline; decode tokens/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
F32_MFMA_PEAK_TFLOPS = 157.3    # dense fp32 matrix
CSRC = os.path.join(ROOT, "linear_attention_02_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hpp", ".hip", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def read_counters(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if current."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_]+)\s*=\s*(\S+)", line)
        if m:
            vals[m.group(1)] = m.group(2)
    if vals.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_copy_peak(torch) -> dict:
    """Bandwidth of a plain 1 GiB device-to-device copy on this GPU (read + write
    bytes over time, median of 10), the practical ceiling the forward's HBM
    fraction is also compared with."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    times = []
    for _ in range(10):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        b.copy_(a)
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    ms = sorted(times)[len(times) // 2]
    del a, b
    return {"GBs": 2 * 4 * n / (ms * 1e-3) / 1e9, "bytes_moved": 2 * 4 * n, "median_ms": ms,
            "what": "torch copy_ of 1 GiB fp32 on the device, read + write bytes"}


def stream_probes(torch) -> dict:
    """Times the streaming probes of libstreamprobes.so (see
    linear_attention_02_amd/probes/stream_probes.hip) on this GPU: the
    sustained rate of each access pattern the attention kernels use, in GB/s
    of bytes read plus written, median of 10 launches after 2 warm-ups."""
    import ctypes
    from linear_attention_02_amd import build as hip_build
    if not os.path.exists(hip_build.PROBES_LIB):
        raise SystemExit("bench.py --probes: libstreamprobes.so is missing (run __graft_entry__.build())")
    P = ctypes.CDLL(hip_build.PROBES_LIB)
    vp, ll, ci = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int
    P.probe_read_lds.argtypes = [vp, ll, ci, vp, vp]
    P.probe_copy.argtypes = [vp, vp, ll, ci, ci, vp]
    P.probe_write.argtypes = [vp, ll, ci, ci, vp]
    P.probe_mix31.argtypes = [vp, vp, vp, vp, ll, ci, ci, vp]
    P.probe_mix31_lds.argtypes = [vp, vp, vp, vp, ll, ci, vp]
    gib = 1 << 30
    big = torch.empty(2 * gib, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    scratch = torch.zeros(1024, dtype=torch.int32, device="cuda")
    parts = big.view(4, gib // 2)
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn, moved):
        for _ in range(2):
            rc = fn()
            if rc != 0:
                raise RuntimeError(f"probe failed: {rc}")
        times = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ms = sorted(times)[len(times) // 2]
        return {"GBs": moved / (ms * 1e-3) / 1e9, "bytes": moved, "median_ms": ms}

    res = {
        "read_lds_default": timed(lambda: P.probe_read_lds(big.data_ptr(), 2 * gib, 0, scratch.data_ptr(), stream),
                                  2 * gib),
        "read_lds_nontemporal": timed(lambda: P.probe_read_lds(big.data_ptr(), 2 * gib, 1, scratch.data_ptr(),
                                                               stream), 2 * gib),
    }
    # The same reads repeated over buffers that fit the 256 MB last-level cache
    # (MALL): what a re-read of recently read data can gain.
    for mib in (128, 256):
        res[f"read_lds_default_{mib}MiB_repeated"] = timed(
            lambda: P.probe_read_lds(big.data_ptr(), mib << 20, 0, scratch.data_ptr(), stream), mib << 20)
    policies = {0: "plain", 1: "nt_loads", 2: "nt_stores", 3: "nt_both"}

    def best(name, launch, moved, write_only=False):
        """Fastest cache policy and workgroup count of one element probe."""
        runs = {}
        for pol in ((0, 2) if write_only else (0, 1, 2, 3)):
            for blocks in (512, 2048):
                runs[f"{policies[pol]}_b{blocks}"] = timed(lambda: launch(pol, blocks), moved)
        key = max(runs, key=lambda k: runs[k]["GBs"])
        res[name] = dict(runs[key], best_of=key, all_GBs={k: round(v["GBs"]) for k, v in runs.items()})

    best("copy", lambda pol, blocks: P.probe_copy(parts[0].data_ptr(), parts[2].data_ptr(), gib, pol, blocks,
                                                   stream), 2 * gib)
    best("write", lambda pol, blocks: P.probe_write(big.data_ptr(), 2 * gib, pol, blocks, stream), 2 * gib,
         write_only=True)
    best("mix_3_reads_1_write", lambda pol, blocks: P.probe_mix31(parts[0].data_ptr(), parts[1].data_ptr(),
                                                                   parts[2].data_ptr(), parts[3].data_ptr(),
                                                                   gib // 2, pol, blocks, stream), 2 * gib)
    res["mix_3_reads_1_write_walk_shaped"] = timed(
        lambda: P.probe_mix31_lds(parts[0].data_ptr(), parts[1].data_ptr(), parts[2].data_ptr(),
                                  parts[3].data_ptr(), gib // 2, 1024, stream), 2 * gib)
    del big, scratch, parts
    res["what"] = ("streaming probes on 2 GiB of traffic each: LDS-DMA staged reads (16 KB chunks, two in flight "
                   "per wave, 1024 waves), also repeated over 128 and 256 MiB buffers that the last-level cache can "
                   "hold; and, each workgroup streaming one contiguous range, a 16-byte copy, "
                   "16-byte writes, and three 16-byte reads per 16-byte write (the causal walk's mix), each the "
                   "best of plain and non-temporal loads and stores at 512 and 2048 workgroups; and the same 3:1 "
                   "mix in the causal walk's structure (1024 one-wave workgroups, four per CU, one 24 KB chunk "
                   "of LDS-DMA loads in flight per wave, non-temporal stores, no arithmetic)")
    return res


def two_stream_forward(la, torch, w, reps: int = 20) -> dict:
    """The headline forward as one call against its two batch halves on two
    streams (default priority), each timed over `reps` calls (or pairs) issued
    back to back with preallocated outputs and workspaces: whether one half's
    read-only totals pass can overlap the other half's walk and raise the
    bytes moved per second."""
    from workloads import forward_inputs
    assert w.B == 2
    q, k, v = (t.cuda() for t in forward_inputs(w))
    o = torch.empty_like(v)
    ws = torch.empty(la.workspace_bytes(w.B, w.H, w.N, q.dtype, True), dtype=torch.uint8, device="cuda")
    halves = []
    for i in range(2):
        hws = torch.empty(la.workspace_bytes(1, w.H, w.N, q.dtype, True), dtype=torch.uint8, device="cuda")
        halves.append((q[i:i + 1], k[i:i + 1], v[i:i + 1], o[i:i + 1], hws))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    main = torch.cuda.current_stream()

    def one():
        la.forward(q, k, v, causal=True, out=o, workspace=ws)

    def two():
        for s, (a, b, c, out, hws) in zip(streams, halves):
            la.forward(a, b, c, causal=True, out=out, workspace=hws, stream=s)

    def timed(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main)
        for s in streams:
            s.wait_stream(main)
        for _ in range(n):
            fn()
        for s in streams:
            main.wait_stream(s)
        e1.record(main)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    timed(one, 3)
    timed(two, 3)
    res = {"one_call_ms": timed(one, reps), "two_streams_ms_per_pair": timed(two, reps),
           "what": f"{w.name} as one call, and as its two batch halves on two streams; {reps} calls (pairs) "
                   "back to back, ms per call (pair)"}
    del q, k, v, o, ws, halves
    return res


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_bf16_b2h8n131072")
    ap.add_argument("--decode-steps", type=int, default=None, help="default: the workload's 3072")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-noncausal", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-generation", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens per head of the headline workload the oracle runs on (0 = all)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--segments", type=int, default=0, help="force segments per head (0 = planner)")
    ap.add_argument("--probes", action="store_true",
                    help="also time the streaming probes (libstreamprobes.so): the sustained rate of each access "
                         "pattern the kernels use, measured in the same run")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_forward(la, torch, w, steps, warmup, segments, host_inputs=None):
    """Times `steps` forwards twice on the same stream: first plainly (the step
    time), then with the library's per-kernel HIP events recorded on the launch
    stream (the per-kernel durations; the events add a little time per kernel
    boundary, so the step time is not taken from this pass)."""
    from workloads import forward_inputs
    host = host_inputs if host_inputs is not None else forward_inputs(w)
    q, k, v = (t.cuda() for t in host)
    out = torch.empty_like(v)
    nbytes = la.workspace_bytes(w.B, w.H, w.N, q.dtype, w.causal)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(with_kernel_events: bool) -> float:
        for _ in range(warmup):
            la.forward(q, k, v, causal=w.causal, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        la.timer.reset()
        la.timer.enable(with_kernel_events)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            la.forward(q, k, v, causal=w.causal, out=out, workspace=ws, stream=stream)
        end.record(stream)
        torch.cuda.synchronize()
        la.timer.enable(False)
        return start.elapsed_time(end) / steps

    ms = timed(False)
    ms_events = timed(True)
    kernels = {}
    for name in la.timer.names():
        kms, n = la.timer.read(name)
        kernels[name] = {"avg_us": 1000.0 * kms / max(n, 1), "launches": n}
    del q, k, v, out, ws
    return ms, kernels, ms_events


def time_forward_cold(la, torch, w, iters=20):
    """One forward per iteration, each after reading a 512 MB scratch buffer
    (outside the timed events) so that neither L2 nor the 256 MB last-level
    cache holds the inputs.  A read rather than a write: a written scrub
    leaves dirty lines whose write-back would be charged to the timed call.
    Returns the median and minimum in ms."""
    from workloads import forward_inputs
    q, k, v = (t.cuda() for t in forward_inputs(w))
    out = torch.empty_like(v)
    ws = torch.empty(max(la.workspace_bytes(w.B, w.H, w.N, q.dtype, w.causal), 1), dtype=torch.uint8, device="cuda")
    scrub = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    times = []
    for i in range(iters + 2):
        torch.sum(scrub, dim=0, out=sink)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        la.forward(q, k, v, causal=w.causal, out=out, workspace=ws)
        end.record()
        torch.cuda.synchronize()
        if i >= 2:
            times.append(start.elapsed_time(end))
    times.sort()
    del q, k, v, out, ws, scrub
    return {"median_ms": times[len(times) // 2], "min_ms": times[0], "iters": iters,
            "protocol": "512 MB scrub read before each timed call"}


def small_call_record(la, torch, w, steps=200):
    """A small forward (the fp32 B=1, H=1, N=256 workload): time per call of
    back-to-back Python calls (host-inclusive), device time per call from one
    replay of a HIP graph holding `steps` calls, and single cold calls."""
    from workloads import forward_inputs
    q, k, v = (t.cuda() for t in forward_inputs(w))
    out = torch.empty_like(v)
    ws = torch.empty(max(la.workspace_bytes(w.B, w.H, w.N, q.dtype, w.causal), 1), dtype=torch.uint8, device="cuda")

    def call():
        la.forward(q, k, v, causal=w.causal, out=out, workspace=ws)

    for _ in range(10):
        call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(end) / steps
    del graph
    cold = time_forward_cold(la, torch, w)
    eb = 2 if w.dtype == "bf16" else 4
    head_tokens = w.B * w.H * w.N
    alg_bytes = head_tokens * 4 * 64 * eb
    alg_flops = head_tokens * 4 * 64 * 64
    peak = F32_MFMA_PEAK_TFLOPS if w.dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
    return {"workload": w.name, "segments_per_head": la.plan_segments(w.B, w.H, w.N, q.dtype, w.causal),
            "us_per_call_eager": 1000.0 * eager_ms, "us_per_call_device": 1000.0 * graph_ms,
            "tokens_per_s_eager": w.tokens / (eager_ms / 1000.0),
            "tokens_per_s_device": w.tokens / (graph_ms / 1000.0),
            "cold_us_median": 1000.0 * cold["median_ms"], "tokens_per_s_cold": w.tokens / (cold["median_ms"] / 1000.0),
            "algorithmic_bytes": alg_bytes, "frac_hbm_device": alg_bytes / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_TFLOPs_device": alg_flops / (graph_ms * 1e-3) / 1e12,
            "frac_mfma_peak_device": alg_flops / (graph_ms * 1e-3) / 1e12 / peak,
            "mfma_peak_TFLOPs": peak,
            "note": "eager: back-to-back Python calls (includes the binding's host time); device: one replay of a "
                    "HIP graph holding the calls; cold: single calls after a 512 MB scrub read; a launch-latency-"
                    "bound size, far below any roofline"}


def time_decode_kernel(la, torch, w, steps=256):
    """Average duration of the decode kernel alone (library HIP events around
    each launch) over `steps` eager steps on the workload's heads."""
    from workloads import decode_inputs
    S = torch.zeros((w.heads, w.C, w.M), dtype=torch.float32, device="cuda")
    z = torch.zeros((w.heads, w.C), dtype=torch.float32, device="cuda")
    out = torch.empty((w.heads, w.M), dtype=torch.float32, device="cuda")
    inputs = [tuple(x.cuda() for x in decode_inputs(w, t)) for t in range(8)]
    for t in range(4):
        la.decode_step(S, z, *inputs[t % 8], out=out)
    torch.cuda.synchronize()
    la.timer.reset()
    la.timer.enable(True)
    for t in range(steps):
        la.decode_step(S, z, *inputs[t % 8], out=out)
    torch.cuda.synchronize()
    la.timer.enable(False)
    ms, n = la.timer.read(f"decode_step_{w.dtype}")
    del S, z, out, inputs
    return 1000.0 * ms / max(n, 1)


def time_backward(la, torch, w, steps, warmup):
    """Times `steps` backward calls like time_forward: plainly, then with the
    library's per-kernel events."""
    from workloads import backward_inputs
    q, k, v, g = (t.cuda() for t in backward_inputs(w))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = la.backward_workspace_bytes(w.B, w.H, w.N, q.dtype, w.causal)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        la.backward(q, k, v, g, causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)

    def timed(with_kernel_events: bool) -> float:
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        la.timer.reset()
        la.timer.enable(with_kernel_events)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            call()
        end.record(stream)
        torch.cuda.synchronize()
        la.timer.enable(False)
        return start.elapsed_time(end) / steps

    ms = timed(False)
    ms_events = timed(True)
    kernels = {}
    for name in la.timer.names():
        kms, n = la.timer.read(name)
        kernels[name] = {"avg_us": 1000.0 * kms / max(n, 1), "launches": n}
    del q, k, v, g, dq, dk, dv, ws
    return ms, kernels, ms_events


def time_train_step(la, torch, w, steps, warmup):
    """Forward then backward reusing the forward's segment states, per step."""
    from workloads import backward_inputs
    q, k, v, g = (t.cuda() for t in backward_inputs(w))
    o = torch.empty_like(v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(la.backward_workspace_bytes(w.B, w.H, w.N, q.dtype, w.causal), 1), dtype=torch.uint8,
                     device="cuda")

    def call():
        la.forward(q, k, v, causal=w.causal, out=o, workspace=ws)
        la.backward(q, k, v, g, causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=ws, after_forward=True)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del q, k, v, g, o, dq, dk, dv, ws
    return ms


def time_train_pair(la, torch, w, steps, warmup):
    """linattn_forward_train then linattn_backward_train: the forward alone,
    the backward alone (it only reads what the forward saved, so it can be
    repeated after one forward), the pair per step, and per-kernel times from
    the library's events (a separate loop)."""
    from workloads import backward_inputs
    q, k, v, g = (t.cuda() for t in backward_inputs(w))
    o = torch.empty_like(v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(la.train_workspace_bytes(w.B, w.H, w.N, q.dtype, w.causal), 1), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    fwd = lambda: la.forward_train(q, k, v, causal=w.causal, out=o, workspace=ws, stream=stream)
    bwd = lambda: la.backward_train(q, k, v, o, g, ws, causal=w.causal, dq=dq, dk=dk, dv=dv, stream=stream)

    def pair():
        fwd()
        bwd()

    def timed(fn, with_kernel_events=False) -> float:
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        la.timer.reset()
        la.timer.enable(with_kernel_events)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        la.timer.enable(False)
        return start.elapsed_time(end) / steps

    rec = {"forward_ms": timed(fwd), "backward_ms": None, "pair_ms": timed(pair)}
    fwd()
    rec["backward_ms"] = timed(bwd)
    timed(pair, with_kernel_events=True)
    rec["kernels"] = {}
    for name in la.timer.names():
        kms, n = la.timer.read(name)
        rec["kernels"][name] = {"avg_us": 1000.0 * kms / max(n, 1), "launches": n}
    del q, k, v, g, o, dq, dk, dv, ws
    return rec


def backward_record(la, torch, w, steps, warmup):
    ms, kernels, ms_events = time_backward(la, torch, w, steps, warmup)
    train_ms = time_train_step(la, torch, w, steps, warmup)
    train = time_train_pair(la, torch, w, steps, warmup)
    eb = 2 if w.dtype == "bf16" else 4
    head_tokens = w.B * w.H * w.N
    row = 64 * eb
    alg = head_tokens * 7 * row  # read Q, K, V, dO; write dQ, dK, dV
    rec = {"workload": w.name, "ms": ms, "ms_with_kernel_events": ms_events,
           "forward_plus_backward_after_forward_ms": train_ms,
           "tokens_per_s": w.tokens / (ms / 1000.0), "algorithmic_bytes": alg,
           "achieved_GBs": alg / (ms * 1e-3) / 1e9, "frac_hbm": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "kernels": kernels}
    # The training pair: linattn_backward_train after linattn_forward_train
    # (bf16 causal: the saved-forward one-pass backward).
    bt = train["backward_ms"]
    rec["train_pair"] = dict(train, backward_tokens_per_s=w.tokens / (bt / 1000.0),
                             backward_frac_hbm=alg / (bt * 1e-3) / 1e9 / HBM_PEAK_GBS)
    # Per-kernel rooflines on the bytes each kernel must move in this design:
    # walk_f reads Q, K, V, dO and writes dQ and one 8-byte pair per token;
    # walk_r reads Q, K, V, dO and the pairs and writes dK, dV.
    per_token = {f"bwd_walk_f_{w.dtype}": 5 * row + 8, f"bwd_walk_r_{w.dtype}": 6 * row + 8,
                 f"bwd_nc_a_{w.dtype}": 3 * row + 8, f"bwd_nc_b_{w.dtype}": 4 * row}
    # Saved-forward backward: the totals read Q, dO, O and 1/den and write the
    # pairs (1/den, b); the walk reads Q, K, V, dO and the pairs and writes
    # dQ, dK, dV.
    per_token_train = {"bwd_saved_totals_bf16": 3 * row + 4 + 8, "bwd_saved_walk_bf16": 7 * row + 8,
                       "causal_walk_save_bf16": 4 * row + 4}
    roof = {}
    for name, b in per_token.items():
        if name in kernels:
            us = kernels[name]["avg_us"]
            gbs = head_tokens * b / (us * 1e-6) / 1e9
            roof[name] = {"bytes_per_launch": head_tokens * b, "avg_launch_us": us, "achieved_GBs": gbs,
                          "frac_hbm": gbs / HBM_PEAK_GBS}
    rec["kernel_rooflines"] = roof
    troof = {}
    for name, b in per_token_train.items():
        if name in train["kernels"]:
            us = train["kernels"][name]["avg_us"]
            gbs = head_tokens * b / (us * 1e-6) / 1e9
            troof[name] = {"bytes_per_launch": head_tokens * b, "avg_launch_us": us, "achieved_GBs": gbs,
                           "frac_hbm": gbs / HBM_PEAK_GBS}
    rec["train_pair"]["kernel_rooflines"] = troof
    return rec


def sequence_sweep(la, torch, steps, warmup, B=1, H=8, exps=range(9, 17)):
    """Forward and forward+backward time and peak device memory against N
    (causal, bf16, B=1, H=8, C=M=64): the pages' memory/time sweep over
    sequence lengths 2^9..2^16, for this library's attention alone.  The
    forward+backward is timed twice: linattn_forward + linattn_backward, and
    the training pair linattn_forward_train + linattn_backward_train."""
    from workloads import draw_grad_output, draw_qkv
    rows = []
    for e in exps:
        N = 1 << e
        q, k, v = (t.cuda() for t in draw_qkv(B, H, N, 64, 64, "bf16", seed=4000 + e))
        g = draw_grad_output(B, H, N, 64, "bf16", 4000 + e).cuda()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        o = la.forward(q, k, v, causal=True)
        grads = la.backward(q, k, v, g, causal=True)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        del o, grads
        fwd_ws = torch.empty(max(la.workspace_bytes(B, H, N, torch.bfloat16, True), 1), dtype=torch.uint8,
                             device="cuda")
        bwd_ws = torch.empty(max(la.backward_workspace_bytes(B, H, N, torch.bfloat16, True), 1),
                             dtype=torch.uint8, device="cuda")
        o = torch.empty_like(v)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

        def fwd():
            la.forward(q, k, v, causal=True, out=o, workspace=fwd_ws)

        def fwd_bwd():
            fwd()
            la.backward(q, k, v, g, causal=True, dq=dq, dk=dk, dv=dv, workspace=bwd_ws)

        # The training pair (what the autograd node runs): forward_train, then
        # backward_train on its output and workspace.
        torch.cuda.synchronize()
        base_t = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        o_t, ws_t = la.forward_train(q, k, v, causal=True)
        grads = la.backward_train(q, k, v, o_t, g, ws_t, causal=True)
        torch.cuda.synchronize()
        peak_train = torch.cuda.max_memory_allocated() - base_t
        del grads

        def train():
            la.forward_train(q, k, v, causal=True, out=o_t, workspace=ws_t)
            la.backward_train(q, k, v, o_t, g, ws_t, causal=True, dq=dq, dk=dk, dv=dv)

        res = {"N": N}
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        for key, fn in (("fwd_ms", fwd), ("fwd_bwd_ms", fwd_bwd), ("train_pair_ms", train)):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            for _ in range(steps):
                fn()
            end.record()
            torch.cuda.synchronize()
            res[key + "_eager"] = start.elapsed_time(end) / steps
            # The same `steps` calls captured in one HIP graph and replayed
            # once: device time without the Python binding's per-call host
            # overhead, which the eager loop pays at small N.
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                for _ in range(steps):
                    fn()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            start.record()
            graph.replay()
            end.record()
            torch.cuda.synchronize()
            res[key] = start.elapsed_time(end) / steps
            del graph
        res["peak_bytes_fwd_bwd"] = int(peak)
        res["peak_bytes_train_pair"] = int(peak_train)
        res["input_bytes"] = int(4 * q.numel() * 2)
        rows.append(res)
        del q, k, v, g, o, dq, dk, dv, fwd_ws, bwd_ws, o_t, ws_t
    return {"shape": f"causal bf16 B={B} H={H} C=M=64", "rows": rows,
            "peak_note": "device memory allocated during one forward + backward call beyond the inputs "
                         "(O, dQ, dK, dV and both workspaces); peak_bytes_train_pair: the same for "
                         "forward_train + backward_train (O, dQ, dK, dV and the train workspace)",
            "time_note": "fwd_ms, fwd_bwd_ms (forward + backward), train_pair_ms (forward_train + "
                         "backward_train): one replay of a HIP graph holding the timed calls, per call "
                         "(device time); *_eager: a loop of Python calls"}


def time_generation(torch, cfg, dtype):
    """Greedy generation of cfg.steps tokens for cfg.batch sequences with the
    random-weight shell, one HIP-graph replay per step; returns images/s and
    ms per step."""
    from linear_attention_02_amd.generation import GenerationShell
    from workloads import draw_shell_weights
    sh = GenerationShell(draw_shell_weights(cfg), cfg.layers, cfg.d_model, cfg.heads, cfg.batch, dtype=dtype)
    sh.capture()
    first = torch.zeros(cfg.batch, dtype=torch.int64)
    sh.generate(16, first)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    sh.generate(cfg.steps, first)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ok = bool(torch.isfinite(sh.logits).all())
    del sh
    return {"images_per_s": cfg.batch / (ms / 1000.0), "ms_per_step": ms / cfg.steps, "total_s": ms / 1000.0,
            "finite": ok}


def time_decode(la, torch, w, steps):
    from workloads import decode_inputs
    heads = w.heads
    log(f"decode: drawing {steps} steps of q/k/v for {heads} heads")
    qs = torch.empty((steps, heads, w.C), dtype=torch.float32)
    ks = torch.empty_like(qs)
    vs = torch.empty((steps, heads, w.M), dtype=torch.float32)
    for t in range(steps):
        q, k, v = decode_inputs(w, t)
        qs[t], ks[t], vs[t] = q, k, v
    qs, ks, vs = qs.cuda(), ks.cuda(), vs.cuda()
    outs = torch.empty((steps, heads, w.M), dtype=torch.float32, device="cuda")
    S = torch.zeros((heads, w.C, w.M), dtype=torch.float32, device="cuda")
    z = torch.zeros((heads, w.C), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    # Warm up on the capture stream, then capture the whole step loop.
    with torch.cuda.stream(stream):
        for t in range(3):
            la.decode_step(S, z, qs[t], ks[t], vs[t], out=outs[t], stream=stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for t in range(steps):
            la.decode_step(S, z, qs[t], ks[t], vs[t], out=outs[t], stream=torch.cuda.current_stream())
    S.zero_()
    z.zero_()
    torch.cuda.synchronize()
    g.replay()  # one untimed replay
    torch.cuda.synchronize()
    S.zero_()
    z.zero_()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    del g
    return total_ms


def cpu_baseline(w, sample_tokens, host_inputs):
    import oracle
    from workloads import to_oracle_array
    n = w.N if sample_tokens <= 0 else min(sample_tokens, w.N)
    q, k, v = (to_oracle_array(t[:, :, :n].contiguous()) for t in host_inputs)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.forward_recurrent(q, k, v, causal=w.causal, threads=threads)
    dt = time.perf_counter() - t0
    # The same oracle on one core, over the first n1 tokens of every head.
    n1 = min(n, 8192)
    q1, k1, v1 = (to_oracle_array(t[:, :, :n1].contiguous()) for t in host_inputs)
    t1 = time.perf_counter()
    oracle.forward_recurrent(q1, k1, v1, causal=w.causal, threads=1)
    d1 = time.perf_counter() - t1
    single = {"value": w.B * n1 / d1, "unit": "tokens/s", "cores": 1, "seconds": d1,
              "sample": f"first {n1} tokens of every head of {w.name}"}
    return {"value": w.B * n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": dt, "single_core": single,
            "sample": f"fp64 C oracle (causal recurrence, O(N) per head) on the first {n} of {w.N} tokens of every "
                      f"head of {w.name} (B={w.B}, H={w.H}, same host inputs as the GPU run); tokens/s counts "
                      f"B*{n} positions over the wall time, threads over (batch, head)"}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Heads shard across GPUs with no communication (each GPU would run this library on its share).", file=sys.stderr)
        return 2
    import torch

    import linear_attention_02_amd as la
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    la.lib()
    if args.segments:
        la.set_segments(args.segments)
    w = WORKLOADS[args.workload]
    from workloads import forward_inputs
    host_inputs = forward_inputs(w)
    log(f"forward {w.name}: steps={args.steps} warmup={args.warmup}")
    ms, kernels, ms_events = time_forward(la, torch, w, args.steps, args.warmup, args.segments, host_inputs)
    tokens_per_s = w.tokens / (ms / 1000.0)
    eb = 2 if w.dtype == "bf16" else 4
    head_tokens = w.B * w.H * w.N
    alg_bytes = head_tokens * (w.C + w.C + w.M + w.M) * eb  # read Q, K, V; write O
    alg_flops = head_tokens * 4 * w.C * w.M                  # state write 2CM + read 2CM per head-token
    dom = f"causal_walk_{w.dtype}" if w.causal else f"noncausal_read_{w.dtype}"
    dom_us = kernels.get(dom, {}).get("avg_us", float("nan"))
    achieved = alg_bytes / (dom_us * 1e-6) / 1e9
    traffic = read_counters(dom, w.name)
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "C": w.C, "M": w.M, "causal": w.causal,
                   "segments_per_head": la.plan_segments(w.B, w.H, w.N, torch.bfloat16, w.causal),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_us": dom_us,
                     "whole_call": {"what": "the same algorithmic bytes over the whole forward call "
                                            "(every kernel of the call and the gaps between them)",
                                    "achieved": alg_bytes / (ms * 1e-3) / 1e9,
                                    "frac": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "ms": ms}},
        "forward_call": {"achieved_GBs": alg_bytes / (ms * 1e-3) / 1e9,
                         "frac_hbm": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "alg_TFLOPs": alg_flops / (ms * 1e-3) / 1e12,
                         "frac_bf16_mfma": alg_flops / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS},
        "kernels": kernels,
        "ms_per_step_with_kernel_events": ms_events,
    }
    log(f"forward {w.name}: cold-cache calls")
    result["forward_call"]["cold"] = time_forward_cold(la, torch, w)
    log("measured copy peak")
    copy_peak = measured_copy_peak(torch)
    result["hbm_measured_copy"] = copy_peak
    result["roofline"]["frac_of_measured_copy"] = achieved / copy_peak["GBs"]
    result["forward_call"]["frac_of_measured_copy"] = result["forward_call"]["achieved_GBs"] / copy_peak["GBs"]
    if args.probes:
        log("streaming probes")
        probes = stream_probes(torch)
        result["stream_probes"] = probes
        # The walk moves three reads to one write: its rate against the probe
        # of that mix measured now, on this device.
        result["roofline"]["frac_of_probe_mix31"] = achieved / probes["mix_3_reads_1_write"]["GBs"]
        log("two-stream forward")
        probes["two_stream_forward"] = two_stream_forward(la, torch, w)
    if not args.no_noncausal:
        for key, name in (("causal_cifar_shaped", "causal_bf16_b16h8n3072"), ("noncausal", "noncausal_bf16_b8h8n4096")):
            wn = WORKLOADS[name]
            log(f"forward {wn.name}")
            nms, nk, _ = time_forward(la, torch, wn, max(10, args.steps), args.warmup, args.segments)
            nbytes = wn.B * wn.H * wn.N * 256 * 2
            cold = time_forward_cold(la, torch, wn)
            cold["achieved_GBs"] = nbytes / (cold["median_ms"] * 1e-3) / 1e9
            cold["frac_hbm"] = cold["achieved_GBs"] / HBM_PEAK_GBS
            result[key] = {"workload": wn.name, "ms": nms, "tokens_per_s": wn.tokens / (nms / 1000.0),
                           "achieved_GBs": nbytes / (nms * 1e-3) / 1e9,
                           "frac_hbm": nbytes / (nms * 1e-3) / 1e9 / HBM_PEAK_GBS, "kernels": nk,
                           "warm_note": "ms is back-to-back (inputs may stay in the last-level cache)",
                           "cold": cold}
    if not args.no_noncausal:
        w1 = WORKLOADS["causal_f32_b1h1n256"]
        log(f"forward {w1.name}")
        result["config_1"] = small_call_record(la, torch, w1)
    if not args.no_backward:
        result["backward"] = {}
        for name in (w.name, "causal_bf16_b16h8n3072", "noncausal_bf16_b8h8n4096"):
            wb = WORKLOADS[name]
            log(f"backward {wb.name}")
            result["backward"][wb.name] = backward_record(la, torch, wb, max(10, args.steps // 2), args.warmup)
    if not args.no_sweep:
        log("sequence-length sweep")
        result["sequence_sweep"] = sequence_sweep(la, torch, 10, 2)
    if not args.no_generation:
        from workloads import SHELLS
        cfg = SHELLS["shell_l12_d512_h8_b256_3072steps"]
        gen = {"workload": cfg.name, "layers": cfg.layers, "d_model": cfg.d_model, "heads": cfg.heads,
               "batch": cfg.batch, "steps": cfg.steps,
               "note": "random weights; greedy decoding; one HIP-graph replay per step; attention through "
                       "linattn_decode_step, dense parts through library GEMMs; the pages' 17.85 images/s "
                       "(2020 hardware, trained CIFAR-10 model) is context, not a comparable target"}
        for key, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
            log(f"generation {cfg.name} {key}")
            gen[key] = time_generation(torch, cfg, dt)
        result["generation"] = gen
    if not args.no_decode:
        wd = WORKLOADS["decode_f32_s256h8_3072steps"]
        steps = args.decode_steps or wd.steps
        log(f"decode {wd.name}: {steps} steps")
        total = time_decode(la, torch, wd, steps)
        per_step = total / steps
        state_bytes = wd.heads * (wd.C * wd.M + wd.C) * 4 * 2
        io_bytes = wd.heads * (wd.C + wd.C + wd.M + wd.M) * 4
        result["decode"] = {"workload": wd.name, "steps": steps, "us_per_step": per_step * 1000.0,
                            "tokens_per_s": wd.sequences * steps / (total / 1000.0),
                            "state_GBs": state_bytes / (per_step * 1e-3) / 1e9,
                            "frac_hbm_state": state_bytes / (per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "bytes_per_step": state_bytes + io_bytes,
                            "note": "one kernel per step, 3072 launches replayed from one HIP graph; the 34 MB "
                                    "state can stay in the MI355X's 256 MB last-level cache between steps"}
        kus = time_decode_kernel(la, torch, wd)
        result["decode"]["kernel_only_us"] = kus
        result["decode"]["kernel_only_state_GBs"] = state_bytes / (kus * 1e-6) / 1e9
        # The same step with 8x the sequences: 272 MB of state, more than the
        # last-level cache holds, so every step moves it through HBM.
        from workloads import DecodeWorkload
        wc = DecodeWorkload("decode_f32_s2048h8_cold", "f32", 8 * wd.sequences, wd.H, 64, seed=wd.seed)
        log(f"decode {wc.name}: {wc.steps} steps")
        total_c = time_decode(la, torch, wc, wc.steps)
        per_c = total_c / wc.steps
        sb = wc.heads * (wc.C * wc.M + wc.C) * 4 * 2
        kc = time_decode_kernel(la, torch, wc, steps=64)
        result["decode"]["cold"] = {"workload": wc.name, "heads": wc.heads, "steps": wc.steps,
                                    "us_per_step": per_c * 1000.0, "kernel_only_us": kc,
                                    "kernel_only_frac_hbm_state": sb / (kc * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                    "tokens_per_s": wc.sequences * wc.steps / (total_c / 1000.0),
                                    "state_GBs": sb / (per_c * 1e-3) / 1e9,
                                    "frac_hbm_state": sb / (per_c * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if args.copy_calibration:
        n = 1 << 28
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = {"read": 4 * n, "write": 4 * n}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens, host_inputs)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
