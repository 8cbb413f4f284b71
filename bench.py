"""Benchmark of the fused AWQ W4A16 linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-secondary] [--copy-calibration]

A step is one awq_gemm call (dispatch by M, packed-weight streaming, unpack,
dequant, multiply-accumulate, reduction, bias, fp16 store) on the workload's
synthetic layer.  Inputs are resident in HBM before timing starts.  The packed
weights are rotated over independent copies totalling >= 512 MB, so every step
reads its weights from HBM rather than from the 256 MB Infinity Cache.  The K
timed steps are captured once into a HIP graph and replayed, so the host's
per-call Python overhead is not what is measured; the graph's output is checked
bit for bit against an eager call.

Prints one JSON line.  `value` is the achieved algorithmic HBM bandwidth (GB/s)
for the bandwidth-bound workloads or TFLOP/s for the compute-bound prefill
workload, over the whole timed region.  `roofline` prices the kernel's average
launch duration (HIP events on the launch stream over the timed region) against
MI355X's peak.  `cpu_baseline` times the CPU oracle on a bounded sample of the
same workload (`cores`: the BLAS threads it used; `host_cores`: the cores this process
may run on).  `read_ceiling` times a plain streaming read of the same byte count (for the
headline and for every other bandwidth-bound workload), and `launch_floor` an empty kernel
of the same grid, i.e. what each dependent launch costs before any work;
`secondary` repeats the timing (not the CPU leg) for every other workload, and for
the large-M (tile family) ones also times the dequantize-then-dense alternative
(awq_dequant_f16 + torch's fp16 GEMM) under the same protocol.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP16_MFMA_PEAK_TFS = 2500.0  # MI355X dense fp16 MFMA
ROTATE_BYTES = 512 << 20     # > 2x the 256 MB Infinity Cache
HEADLINE = "decode_m1_k4096_n4096_g128"
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads (reported under 'secondary' by default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run three 256 MiB device-to-device copies, a plain copy kernel of "
                         "known size that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_weight_only_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not os.path.isfile(os.path.join(csrc, f)):
            continue  # the probe/ subdirectory is not an AWQ kernel
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


SETTLE_S = 0.25  # untimed graph replays before a timed one: clocks and caches settle


_HIP = None


def replay(graph, stream):
    """Launch the captured graph on `stream` with hipGraphLaunch on its executable graph:
    the launch torch's CUDAGraph.replay() makes, without that call's host-side bookkeeping
    (about 8 us per launch, which the wall clock around a 20-call region would count)."""
    global _HIP
    import ctypes
    if _HIP is None:
        lib = ctypes.CDLL("libamdhip64.so")
        lib.hipGraphLaunch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipGraphLaunch.restype = ctypes.c_int
        _HIP = lib
    rc = _HIP.hipGraphLaunch(ctypes.c_void_p(graph.raw_cuda_graph_exec()), ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"hipGraphLaunch returned {rc}")


def settle(graph, stream, torch, seconds=SETTLE_S):
    """Replay `graph` untimed until `seconds` have passed (at least once), so that a short
    timed region (a few steps) measures the steady state rather than the GPU's clock ramp
    after idling.  Returns the number of replays."""
    n = 0
    t0 = time.perf_counter()
    while True:
        with torch.cuda.stream(stream):
            for _ in range(4):
                replay(graph, stream)
        n += 4
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def time_workload(name, steps, warmup, torch, awq, synth, bf16=False):
    """awq_gemm on workload `name`; bf16=True takes bfloat16 x, bias and y (awq_gemm_bf16)."""
    w = synth.WORKLOADS[name]
    d = synth.make_inputs_bf16(w) if bf16 else synth.make_inputs(w)
    dev = torch.device("cuda", 0)
    layer_bytes = d["qweight"].nbytes + d["qzeros"].nbytes + d["scales"].nbytes
    copies = max(1, -(-ROTATE_BYTES // layer_bytes))

    def act(a):
        if a is None:
            return None
        t = torch.from_numpy(a.view(np.int16) if bf16 else a).to(dev)
        return t.view(torch.bfloat16) if bf16 else t
    x = act(d["x"])
    bias = act(d["bias"])
    weights = []
    for i in range(copies):
        # Independent buffers with identical contents: the same layer, fresh addresses.
        weights.append(tuple(torch.from_numpy(d[k]).to(dev) for k in ("qweight", "qzeros", "scales")))
    y = torch.empty((w.M, w.N), dtype=torch.bfloat16 if bf16 else torch.float16, device=dev)
    g = w.group_size
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()

    def step(i):
        qw, qz, sc = weights[i % copies]
        awq.awq_gemm(x, qw, qz, sc, bias, g, out=y)

    with torch.cuda.stream(stream):
        for i in range(max(warmup, 1)):  # eager warm-up; allocates the split-K workspace
            step(i)
        eager = y.clone()
    stream.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            step(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()  # untimed replay through torch: graph upload and first-touch
        ev0.record(stream)  # the events' first record creates them: keep that out of the timing
        ev1.record(stream)
    torch.cuda.synchronize()
    warm_replays = settle(graph, stream, torch)

    # The timed region: barrier, the K calls (one graph launch), barrier.  ev0 is recorded
    # just before it on the same stream, so the event pair brackets the same calls.
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        ev0.record(stream)
        t0 = time.perf_counter()
        replay(graph, stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall_s = t1 - t0
    event_s = ev0.elapsed_time(ev1) / 1e3
    if not torch.equal(y.view(torch.int16), eager.view(torch.int16)):
        raise RuntimeError("graph replay output differs from the eager call")
    del weights
    torch.cuda.empty_cache()
    return dict(workload=w, wall_s=wall_s, event_s=event_s, copies=copies, warm_replays=warm_replays,
                plan=awq.plan(w.M, w.K, w.N, w.group_size))


def time_dequant_dense(name, steps, torch, awq, synth):
    """The pages' large-batch alternative on the same inputs and protocol: awq_dequant_f16
    into one fp16 [K, N] buffer, then torch's dense fp16 GEMM (hipBLASLt) with the bias
    folded in (addmm).  Returns us per call; a comparison point, not the product path."""
    w = synth.WORKLOADS[name]
    d = synth.make_inputs(w)
    dev = torch.device("cuda", 0)
    layer_bytes = d["qweight"].nbytes + d["qzeros"].nbytes + d["scales"].nbytes
    copies = max(1, -(-ROTATE_BYTES // layer_bytes))
    x = torch.from_numpy(d["x"]).to(dev)
    bias = None if d["bias"] is None else torch.from_numpy(d["bias"]).to(dev)
    weights = [tuple(torch.from_numpy(d[k]).to(dev) for k in ("qweight", "qzeros", "scales")) for _ in range(copies)]
    wf = torch.empty((w.K, w.N), dtype=torch.float16, device=dev)
    y = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.Stream(dev)

    def step(i):
        qw, qz, sc = weights[i % copies]
        awq.awq_dequant(qw, qz, sc, w.group_size, out=wf, dtype=torch.float16)
        if bias is None:
            torch.matmul(x, wf, out=y)
        else:
            torch.addmm(bias, x, wf, out=y)

    with torch.cuda.stream(stream):
        for i in range(3):
            step(i)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            step(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        replay(graph, stream)
        ev0.record(stream)  # first records create the events, outside the timing
        ev1.record(stream)
        stream.synchronize()
    settle(graph, stream, torch)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        replay(graph, stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    del weights, graph
    torch.cuda.empty_cache()
    return round(us, 3)


def time_quantize_rtn(K, N, g, sym, steps, torch, awq, synth):
    """The RTN writer on a [K, N] fp16 weight, same protocol (rotated copies, one graph
    replay timed with HIP events on the launch stream).  Algorithmic bytes: the fp16
    weight read once, the packed codes written, plus 2.5 bytes per (group, column)
    of scales and zeros."""
    G = 1 if g == -1 else K // g
    nbytes = K * N * 2 + K * N // 2 + G * N * 2 + G * N // 2
    dev = torch.device("cuda", 0)
    W = torch.from_numpy(synth.make_weights(K, N, seed=1)).to(dev)
    copies = max(1, -(-ROTATE_BYTES // (K * N * 2)))
    ws = [W.clone() for _ in range(copies)]
    outs = [awq.awq_quantize_rtn(ws[i], g, sym) for i in range(copies)]
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()

    def step(i):
        awq.awq_quantize_rtn(ws[i % copies], g, sym, out=outs[i % copies])

    with torch.cuda.stream(stream):
        for i in range(3):
            step(i)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            step(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        replay(graph, stream)
        ev0.record(stream)  # first records create the events, outside the timing
        ev1.record(stream)
        stream.synchronize()
    settle(graph, stream, torch)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        replay(graph, stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    s_per = ev0.elapsed_time(ev1) / 1e3 / steps
    del ws, outs, graph
    torch.cuda.empty_cache()
    gbs = nbytes / s_per / 1e9
    return dict(K=K, N=N, group_size=g, sym=bool(sym), kernel_avg_us=round(s_per * 1e6, 3),
                algorithmic_bytes=nbytes, achieved_gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))


def time_moe(name, steps, torch, awq, synth):
    """awq_moe_gemm on a routed-expert workload, same protocol (expert weights rotated
    over >= 512 MB, one graph replay timed with HIP events).  Algorithmic bytes: the
    packed weights, zeros and scales of every expert that receives a slot, x once and
    y once; FLOPs 2 * slots * K * N."""
    w = synth.MOE_WORKLOADS[name]
    d = synth.make_moe_inputs(w)
    dev = torch.device("cuda", 0)
    active = np.unique(d["expert_ids"]).size
    per_expert = (d["qweight"][0].nbytes + d["qzeros"][0].nbytes + d["scales"][0].nbytes)
    nbytes = active * per_expert + d["x"].nbytes + w.slots * w.N * 2
    flops = 2 * w.slots * w.K * w.N
    copies = max(1, -(-ROTATE_BYTES // (w.E * per_expert)))
    x = torch.from_numpy(d["x"]).to(dev)
    ids = torch.from_numpy(d["expert_ids"].reshape(w.T, w.topk)).to(dev)
    weights = [tuple(torch.from_numpy(d[k]).to(dev) for k in ("qweight", "qzeros", "scales")) for _ in range(copies)]
    y = torch.empty((w.slots, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.Stream(dev)

    def step(i):
        qw, qz, sc = weights[i % copies]
        awq.awq_moe_gemm(x, qw, qz, sc, ids, w.group_size, out=y)

    with torch.cuda.stream(stream):
        for i in range(3):
            step(i)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            step(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        replay(graph, stream)
        ev0.record(stream)  # first records create the events, outside the timing
        ev1.record(stream)
        stream.synchronize()
    settle(graph, stream, torch)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        replay(graph, stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    s_per = ev0.elapsed_time(ev1) / 1e3 / steps
    del weights, graph
    torch.cuda.empty_cache()
    gbs, tfs = nbytes / s_per / 1e9, flops / s_per / 1e12
    mfma_bound = flops / nbytes > (FP16_MFMA_PEAK_TFS * 1e12) / (HBM_PEAK_GBS * 1e9)
    roof = (dict(bound="mfma", achieved=round(tfs, 2), peak=FP16_MFMA_PEAK_TFS, unit="TFLOP/s", frac=round(tfs / FP16_MFMA_PEAK_TFS, 4))
            if mfma_bound else dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                                    frac=round(gbs / HBM_PEAK_GBS, 4)))
    return dict(workload=name, active_experts=int(active), call_us=round(s_per * 1e6, 3), algorithmic_bytes=nbytes,
                flops=flops, roofline=roof,
                note=("one call = skinny kernel batched over experts (+ split reduce), no alignment pass"
                      if w.T <= 16 else "one call = alignment kernel + grouped tile kernel"))


def read_ceiling(nbytes, torch, steps=400):
    """A plain streaming read of the same byte count for comparison: the probe
    library's read kernel (16-byte nontemporal loads, 16 KiB contiguous per
    workgroup, no arithmetic), over the same rotation of >= 512 MB of copies and
    replayed from a HIP graph like the timed steps.  At a few MB per launch it is
    bound by launch and memory latency rather than by HBM bandwidth."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "w4a16_weight_only_amd", "libawq_probe.so"))
    probe.awq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    probe.awq_probe_stream_read.restype = ctypes.c_int
    n = max(16, nbytes // 16 * 16)
    copies = max(1, -(-ROTATE_BYTES // n))
    bufs = [torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(n // 16384 + 1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def go(i):
        st = probe.awq_probe_stream_read(bufs[i % copies].data_ptr(), n, sink.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"awq_probe_stream_read failed: {st}")

    with torch.cuda.stream(stream):
        for i in range(3):
            go(i)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            go(i)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        replay(graph, stream)
        ev0.record(stream)  # first records create the events, outside the timing
        ev1.record(stream)
        stream.synchronize()
    settle(graph, stream, torch)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        replay(graph, stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    del bufs
    torch.cuda.empty_cache()
    return dict(bytes=n, us_per_launch=round(us, 3), gbs=round(n / (us * 1e-6) / 1e9, 1),
                how="libawq_probe.so stream read of the same byte count, rotated, graph-replayed")


def launch_floor(blocks, threads, torch, steps=400):
    """Per-launch time of an empty kernel with the given grid, replayed from a HIP graph
    like the timed steps: what each dependent launch costs on this device before any work
    (the probe library's empty kernel)."""
    import ctypes
    probe = ctypes.CDLL(os.path.join(ROOT, "w4a16_weight_only_amd", "libawq_probe.so"))
    probe.awq_probe_empty.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.awq_probe_empty.restype = ctypes.c_int
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def go():
        st = probe.awq_probe_empty(blocks, threads, sink.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"awq_probe_empty failed: {st}")

    with torch.cuda.stream(stream):
        go()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(steps):
            go()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        replay(graph, stream)
        ev0.record(stream)
        ev1.record(stream)
        stream.synchronize()
    settle(graph, stream, torch)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        replay(graph, stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    return dict(blocks=blocks, threads=threads, us_per_launch=round(us, 3),
                how="libawq_probe.so empty kernel of the same grid, graph-replayed")


def summarize(r, steps):
    w = r["workload"]
    ab = w.algorithmic_bytes()
    fl = w.flops()
    per_launch_s = r["event_s"] / steps
    compute_bound = w.M >= 512
    if compute_bound:
        value = fl * steps / r["wall_s"] / 1e12
        achieved = fl / per_launch_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=FP16_MFMA_PEAK_TFS, unit="TFLOP/s",
                    frac=round(achieved / FP16_MFMA_PEAK_TFS, 4))
        unit = "TFLOP/s"
    else:
        value = ab * steps / r["wall_s"] / 1e9
        achieved = ab / per_launch_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
        unit = "GB/s"
    return value, unit, roof, per_launch_s


def cpu_baseline(name, synth):
    """The CPU oracle on the same workload: a bounded number of full-layer calls."""
    from oracle import awq_ref
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    w = synth.WORKLOADS[name]
    d = synth.make_inputs(w)
    reps = 0
    t0 = time.perf_counter()
    while True:
        awq_ref.gemm_ref(d["x"], d["qweight"], d["qzeros"], d["scales"], d["bias"], w.group_size)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or reps >= 200:  # about 10 s of CPU work
            break
    per = el / reps
    if w.M >= 512:
        value, unit = w.flops() / per / 1e12, "TFLOP/s"
    else:
        value, unit = w.algorithmic_bytes() / per / 1e9, "GB/s"
    host_cores = len(os.sched_getaffinity(0))
    return dict(value=round(value, 4), unit=unit, cores=int(blas_threads), host_cores=host_cores, kind="oracle",
                sample=f"{reps} full calls of the {name} layer (unpack, fp32 dequant, fp64 matmul), "
                       f"{per:.2f} s each; numpy elementwise on 1 thread, BLAS on {blas_threads} of the "
                       f"{host_cores} host cores this process may use")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build runs on a "
              f"single MI355X and has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(1)
    import w4a16_weight_only_amd as awq
    from w4a16_weight_only_amd import synth
    awq.load_library()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    r = time_workload(args.workload, args.steps, args.warmup, torch, awq, synth)
    value, unit, roof, per_launch_s = summarize(r, args.steps)
    digest = kernel_source_digest()
    roof["traffic"] = load_traffic(args.workload, digest)
    w = r["workload"]
    out = {
        "metric": "awq_gemm achieved HBM GB/s (M=1,16) and TFLOP/s (M=2048), % of roofline",
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_s"] / args.steps * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 x / int4 weights / fp32 accumulate",
        "data": "synthetic (seeded; random packed words, fp16 scales U[1e-3,2e-2], x ~ N(0,1))",
        "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "group_size": w.group_size,
                   "bias": w.bias, "algorithmic_bytes": w.algorithmic_bytes(), "flops": w.flops(),
                   "plan": r["plan"], "weight_copies_rotated": r["copies"],
                   "timing": "HIP graph of all steps, wall clock over one replay, after "
                             f"{r['warm_replays']} untimed replays ({SETTLE_S} s) that let clocks settle"},
        "roofline": roof,
        "kernel_avg_us": round(per_launch_s * 1e6, 3),
        "source_digest": digest,
    }
    out["read_ceiling"] = read_ceiling(w.algorithmic_bytes(), torch)
    pg = r["plan"]
    out["launch_floor"] = launch_floor(int(pg["grid"][0]) * int(pg["grid"][1]), int(pg["block"]), torch)
    if not args.no_secondary:
        # Every other workload once, shorter: parity-test shapes, reported for context.
        sec = []
        for name in synth.WORKLOADS:
            if name == args.workload or name.startswith("tiny"):
                continue
            n_steps = min(args.steps, 200)
            rs = time_workload(name, n_steps, 10, torch, awq, synth)
            v, u, rf, pl = summarize(rs, n_steps)
            entry = dict(workload=name, value=round(v, 2), unit=u, kernel_avg_us=round(pl * 1e6, 3),
                         plan=rs["plan"], roofline=rf)
            if rf["bound"] == "hbm":
                entry["read_ceiling"] = read_ceiling(rs["workload"].algorithmic_bytes(), torch, steps=n_steps)
                pg = rs["plan"]
                entry["launch_floor"] = launch_floor(int(pg["grid"][0]) * int(pg["grid"][1]), int(pg["block"]), torch,
                                                     steps=n_steps)
            if rs["plan"]["family"] == "tile":
                dd = time_dequant_dense(name, n_steps, torch, awq, synth)
                entry["dequant_then_dense_us"] = dd  # awq_dequant_f16 + hipBLASLt fp16 GEMM
            sec.append(entry)
        out["secondary"] = sec
        # bfloat16 activations (awq_gemm_bf16) on the same weights.
        bf = []
        for name in ("decode_m1_k4096_n4096_g128", "decode_m16_k4096_n11008_g128", "down_proj_m64_k11008_n4096_g64",
                     "down_proj_m512_k11008_n4096_g64", "prefill_m2048_k4096_n4096_g128"):
            n_steps = min(args.steps, 200)
            rs = time_workload(name, n_steps, 10, torch, awq, synth, bf16=True)
            v, u, rf, pl = summarize(rs, n_steps)
            bf.append(dict(workload=name, value=round(v, 2), unit=u, kernel_avg_us=round(pl * 1e6, 3), roofline=rf))
        out["bf16"] = bf
        # Routed experts (awq_moe_gemm).
        out["moe"] = [time_moe(name, min(args.steps, 50), torch, awq, synth) for name in synth.MOE_WORKLOADS]
        # The RTN writer (fp16 weight -> GEMM pack), HBM-bound.
        out["writer"] = [time_quantize_rtn(K, N, g, sym, min(args.steps, 100), torch, awq, synth)
                         for (K, N, g, sym) in ((4096, 4096, 128, False), (4096, 4096, 128, True),
                                                (4096, 14336, 128, False), (4096, 4096, -1, False),
                                                (11008, 4096, 256, False))]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
