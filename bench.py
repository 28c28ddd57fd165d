#!/usr/bin/env python3
"""Benchmark of the W4A16 group-quantized linear layer on one MI355X.

Default workload (the headline): the decode GEMV C[12288] = Wdeq[12288, 4096]
. x[4096] with int4 weights, fp16 scales, 4-bit zeros, g = 128.  One step is
one call of the layer on one batch (here one activation column), reading
the whole packed matrix once.  The weights are replicated into R device
copies (R * 26 MB > 1 GB, four times the 256 MB last-level cache) and the
steps cycle through them, so every call streams its weights from HBM.
Exactly --steps calls are timed: they are captured in one HIP graph, HIP
events on the launch stream bracket its replay, and a graph of --warmup
untimed calls runs right before it, after --clock-warmup seconds of
untimed calls that bring the clocks up.

Printed (one JSON line): GB/s of algorithmic bytes (packed weights, scales,
zeros, x and C, each counted once) per call, the roofline fraction against
8 TB/s, the large-N GEMM figure at N = 4096 (TFLOP/s against the 2.5 PF/s
fp16 dense peak) as a second measurement, and the CPU oracle timed on a
bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME]
  python bench.py --trace-summary DIR --kernel NAME --last K   (no GPU: the
      last K dispatches of a kernel in a rocprofv3 kernel trace)
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
GROUP = 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CSRC = os.path.join(ROOT, "gemm_w4a16_group_amd", "csrc")
KERNEL_SOURCES = {"skinny_kernel": ("device.hpp", "skinny.hip"),
                  "tiled_kernel": ("device.hpp", "tiled.hip"),
                  "tiled_dx_kernel": ("device.hpp", "tiled.hip")}


def alg_bytes(M, K, N):
    """Algorithmic bytes of one call: each array moved once."""
    G = K // GROUP
    return M * K // 2 + 2 * M * G + M * G // 2 + 2 * K * N + 2 * M * N


def alg_flops(M, K, N):
    return 2 * M * K * N


def sources_sha(kernel):
    """sha256 over the code a kernel is built from: its source file, the
    device helpers and the kernels' argument struct (comments and blank lines
    left out, so that editing a comment does not retire the stored
    counters)."""
    import hashlib
    import re
    h = hashlib.sha256()
    # the kernels' argument struct, from the launcher declarations
    with open(os.path.join(CSRC, "launch.hpp")) as fh:
        m = re.search(r"struct GemmArgs \{.*?\n\};", fh.read(), flags=re.S)
    h.update(re.sub(r"//[^\n]*", "", m.group(0)).encode())
    for f in KERNEL_SOURCES[kernel.split("<")[0]]:
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
        h.update(code.encode())
    return h.hexdigest()


def traffic(kernel, M, K, N):
    """HBM bytes per launch of `kernel` at this shape from the stored rocprofv3
    FETCH_SIZE / WRITE_SIZE counters, each scaled by what the same counter
    reads for a copy kernel of known size; None when no counters were taken
    or the kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = t.get("kernels", {}).get("%s@%dx%dx%d" % (kernel, M, K, N))
    cal = t.get("calibration")
    if not rec or not cal or rec.get("sources_sha256") != sources_sha(kernel):
        return None
    b = rec["fetch_kib"] * 1024 * cal["fetch_factor"] + rec["write_kib"] * 1024 * cal["write_factor"]
    return int(round(b))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed calls (exactly this many)")
    ap.add_argument("--warmup", type=int, default=200, help="untimed calls right before the timed ones")
    # from idle the clocks take a few milliseconds to ramp up and the first
    # thousands of calls run slower: a time-based warm-up always runs first
    ap.add_argument("--clock-warmup", type=float, default=0.5, help="seconds of untimed calls first (>= 0.3)")
    ap.add_argument("--copies", type=int, default=40, help="weight copies cycled through (cold cache)")
    ap.add_argument("--workload", default="gemv_12288x4096",
                    choices=["gemv_12288x4096", "gemv_4096x4096", "decode_linears", "small_n",
                             "large_n", "stack", "gemm_12288x4096_n4096", "copy_calib",
                             "quantize_12288x4096", "prologue", "attention", "tune_table", "decode_step",
                             "read_floor", "read_calib"])
    ap.add_argument("--gemm-iters", type=int, default=20)
    ap.add_argument("--gemm-warmup", type=int, default=1000, help="untimed N = 4096 calls first (about 0.4 s)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--token", action="store_true",
                    help="small_n / large_n: token-major x [N, K] and c [N, M]")
    ap.add_argument("--trace-summary", metavar="DIR_OR_CSV",
                    help="summarize a rocprofv3 kernel trace (no GPU): the last --last dispatches of --kernel")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="write profiles/traffic_counters.{json,md} from counter summaries (no GPU)")
    ap.add_argument("--counter-summary", metavar="DIR_OR_CSV",
                    help="summarize rocprofv3 --pmc counters of --kernel (no GPU)")
    ap.add_argument("--kernel", help="with --trace-summary / --counter-summary: the kernel's full name as "
                                     "rocprofv3 prints it")
    ap.add_argument("--last", type=int, default=0, help="with --trace-summary: dispatches counted from the end")
    args = ap.parse_args()
    args.clock_warmup = max(args.clock_warmup, 0.3)
    return args


class Layer:
    """One weight matrix packed on the device, replicated ``copies`` times."""

    def __init__(self, M, K, wid, proj=0, layer=0, copies=1):
        import torch
        from gemm_w4a16_group_amd import binding as B
        from gemm_w4a16_group_amd import inputs
        self.M, self.K = M, K
        q, s, z = inputs.weights(M, K, wid=wid, layer=layer, proj=proj)
        self.host = (q, s, z)
        qpk, zpk = B.pack(torch.from_numpy(q).cuda(), torch.from_numpy(z).cuda())
        sd = torch.from_numpy(s).cuda()
        self.copies = [(qpk, sd, zpk)]
        for _ in range(copies - 1):
            self.copies.append((qpk.clone(), sd.clone(), zpk.clone()))
        torch.cuda.synchronize()


def capture(calls, stream):
    """Capture a list of zero-argument launch closures into one HIP graph."""
    import torch
    with torch.cuda.stream(stream):
        for c in calls:          # eager run first: allocations, lazy loading
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    return g


def warm_graph(g, stream, seconds):
    """Replay ``g`` untimed for about ``seconds`` (clock ramp-up)."""
    import torch
    t0 = time.time()
    with torch.cuda.stream(stream):
        while time.time() - t0 < seconds:
            for _ in range(4):
                g.replay()
            torch.cuda.synchronize()


def time_graph(g, replays, stream):
    """Milliseconds of ``replays`` graph replays, HIP events on ``stream``."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def timed_calls(calls, steps, warmup, clock_s):
    """Time exactly ``steps`` calls, call i being calls[i % len(calls)] (one
    per weight copy, so that every call streams its weights from HBM).
    Three HIP graphs: one rotation over the copies (replayed for ``clock_s``
    seconds of clock warm-up), ``warmup`` calls and ``steps`` calls.  The
    warm-up graph is enqueued right before the timed one, so that the timed
    calls start without a launch gap; HIP events on the launch stream
    bracket the timed graph.  Returns (ms per call, seconds of clock warm-up,
    one rotation included)."""
    import torch
    stream = torch.cuda.Stream()
    rot = capture(calls, stream)
    timed = capture([calls[i % len(calls)] for i in range(steps)], stream)
    warm = capture([calls[(steps + i) % len(calls)] for i in range(warmup)], stream) if warmup > 0 else rot
    t0 = time.time()
    warm_graph(rot, stream, clock_s)
    # each graph replayed once before it is timed (the first replay of a
    # graph also sets it up on the device)
    with torch.cuda.stream(stream):
        warm.replay()
        timed.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        # one more rotation first: the host enqueues the rest while it runs,
        # so that the timed graph is queued before the start event is reached
        rot.replay()
        warm.replay()
        start.record(stream)
        timed.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, time.time() - t0


def gemv_rotation(M, K, wid, copies, steps, warmup, plan=None, clock_s=0.5):
    """Time exactly `steps` calls cycling over `copies` weight copies, after
    `warmup` untimed calls and a clock warm-up.  Returns (ms per call, plan
    dict, seconds of clock warm-up, the weights, x, the first output)."""
    import torch
    from gemm_w4a16_group_amd import binding as B
    from gemm_w4a16_group_amd import inputs
    lay = Layer(M, K, wid, copies=copies)
    x = torch.from_numpy(inputs.activations(K, 1, wid=wid)).cuda()
    outs = [torch.empty((M, 1), dtype=torch.float16, device="cuda") for _ in range(copies)]
    calls = [(lambda c=c, o=o: B.gemm(c[0], c[1], c[2], x, out=o, plan=plan))
             for c, o in zip(lay.copies, outs)]
    ms, clock = timed_calls(calls, steps, warmup, clock_s)
    return ms, B.plan_default(M, 1, K).as_dict(), clock, lay, x, outs[0]


def gemm_large(M, K, N, wid, iters, warmup=1000):
    """Eager timing of the large-N GEMM (each call is hundreds of us), after
    ``warmup`` untimed calls."""
    import torch
    from gemm_w4a16_group_amd import binding as B
    from gemm_w4a16_group_amd import inputs
    lay = Layer(M, K, wid)
    qpk, sd, zpk = lay.copies[0]
    x = torch.from_numpy(inputs.activations(K, N, wid=wid)).cuda()
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            B.gemm(qpk, sd, zpk, x, out=out)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(iters):
            B.gemm(qpk, sd, zpk, x, out=out)
        end.record(stream)
    end.synchronize()
    ms = start.elapsed_time(end) / iters
    return ms, B.plan_default(M, N, K).as_dict()


def cpu_baseline(M, K, seconds, wid):
    """The oracle on the same workload, repeated for about ``seconds``."""
    import numpy as np
    import oracle.w4a16 as ora
    from gemm_w4a16_group_amd import inputs
    q, s, z = inputs.weights(M, K, wid=wid)
    X = inputs.activations(K, 1, wid=wid)
    qpk, zpk = ora.pack(q, z)
    try:
        from threadpoolctl import threadpool_info
        blas = [(d.get("internal_api"), d.get("num_threads")) for d in threadpool_info()
                if d.get("user_api") == "blas"]
    except Exception:
        blas = []
    threads = max([t for _, t in blas] or [1])
    n = 0
    t0 = time.perf_counter()
    while True:
        ora.reference(qpk, s, zpk, X)
        n += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n >= 2) or n >= 200:
            break
    per = el / n
    return {
        "value": alg_bytes(M, K, 1) / per / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": "%d full calls of the fp64 numpy oracle on %dx%d, N=1 (%.2f s each; dequant "
                  "single-threaded numpy, product %s with %d threads, %d host cores visible)"
                  % (n, M, K, per, "/".join(str(b[0]) for b in blas) or "BLAS", threads,
                     len(os.sched_getaffinity(0))),
    }


def gemm_secondary(iters, warmup):
    """The N = 4096 GEMM figure (one call; the tiled kernel reads X [K, N] in place,
    so the call is that one launch)."""
    from gemm_w4a16_group_amd import binding as B
    M, K, N = 12288, 4096, 4096
    gms, gplan = gemm_large(M, K, N, 4, iters, warmup)
    tf = alg_flops(M, K, N) / (gms * 1e-3) / 1e12
    kern = B.kernel_name(M, N, K)
    return {
        "metric": "W4A16 GEMM TFLOP/s (12288x4096, N=4096)", "value": round(tf, 2),
        "unit": "TFLOP/s", "ms_per_call": round(gms, 4), "plan": gplan,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / FP16_PEAK_TFLOPS, 4),
                     "traffic": traffic(kern, M, K, N), "kernel": kern,
                     "flops_per_launch": alg_flops(M, K, N),
                     "timed": "whole call: %s%s" % (
                         "" if "_dx_" in kern else "xpack_col_kernel (activation re-layout) + ", kern)}}


def headline(args):
    import torch
    from gemm_w4a16_group_amd import binding as B
    M, K, N = 12288, 4096, 1
    wid = 3
    ms, plan, clock, *_ = gemv_rotation(M, K, wid, args.copies, args.steps, args.warmup, clock_s=args.clock_warmup)
    steps = args.steps
    b = alg_bytes(M, K, N)
    gbs = b / (ms * 1e-3) / 1e9
    kern = B.kernel_name(M, N, K)
    line = {
        "metric": "W4A16 GEMV HBM GB/s (12288x4096,N=1) + GEMM TFLOPS at N=4096; % roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "gemv_12288x4096_n1", "M": M, "K": K, "N": N, "group_size": GROUP,
                   "weights": "int4 packed, fp16 scale + 4-bit zero per 128",
                   "cold_cache_copies": args.copies,
                   "timing": "HIP graph of exactly %d calls cycling over %d weight copies, HIP events on the "
                             "launch stream; %d untimed calls right before, after %.2f s of clock warm-up"
                             % (steps, args.copies, args.warmup, clock),
                   "clock_warmup_s": round(clock, 3), "plan": plan},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic(kern, M, K, N),
                     "kernel": kern, "bytes_per_launch": b,
                     "us_per_launch": round(ms * 1e3, 3)},
    }
    if not args.no_gemm:
        line["secondary"] = gemm_secondary(args.gemm_iters, args.gemm_warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(M, K, args.cpu_seconds, wid)
    print(json.dumps(line), flush=True)


def read_calib():
    """The streaming-read probe over one 512 MiB buffer, five launches: the
    reference the rocprofv3 read counter (FETCH_SIZE) is scaled by, since it
    reads exactly its buffer with 1 KB runs per load instruction, as the
    weight streams do."""
    import torch
    from gemm_w4a16_group_amd import binding as B
    nb = 512 << 20
    buf = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for _ in range(5):
        B.stream_read(buf, waves=8, loads=4)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "read_calib", "launches": 5, "bytes_read_per_launch": nb}), flush=True)


def copy_calib():
    """A plain fp16 copy kernel of known size (reads and writes 512 MiB each
    launch): the reference that rocprofv3 FETCH_SIZE / WRITE_SIZE are scaled
    by."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copy_calib", "launches": 5, "bytes_read_per_launch": 2 * n,
                      "bytes_written_per_launch": 2 * n}), flush=True)


def extra(args):
    """Other workloads, one JSON line each (for tuning and the design notes)."""
    import numpy as np
    import torch
    from gemm_w4a16_group_amd import binding as B
    from gemm_w4a16_group_amd import inputs
    rows = []
    if args.workload == "copy_calib":
        copy_calib()
        return
    if args.workload == "read_calib":
        read_calib()
        return
    if args.workload == "read_floor":
        # the streaming-read probe (one launch reads a buffer once) over
        # buffers of each decode linear's algorithmic bytes at N = 1 and two
        # larger sizes, copies cycled through as in the GEMV (cold cache): in
        # the GEMV's launch shape (eight waves per workgroup, 4 KB per wave)
        # and, at the 12288x4096 size, across launch shapes
        sizes = [("12288x4096", alg_bytes(12288, 4096, 1), [(w, l) for w in (4, 8, 16) for l in (1, 2, 4, 8, 16)])]
        sizes += [(name + "_%dx%d" % (M, K), alg_bytes(M, K, 1), [(8, 4)]) for (name, M, K) in inputs.LLAMA7B_PROJ]
        sizes += [("100MiB", 100 << 20, [(8, 4)]), ("200MiB", 200 << 20, [(8, 4)])]
        for name, nb, shapes in sizes:
            nb = nb // 16 * 16
            cps = max(4, -(-int(1.1e9) // nb))
            bufs = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(cps)]
            for waves, loads in shapes:
                words = int(B.lib().w4a16_stream_read_sink_words(nb, waves, loads))
                sinks = [torch.empty(words, dtype=torch.int32, device="cuda") for _ in range(cps)]
                calls = [(lambda b=b, k=k, w=waves, l=loads: B.stream_read(b, sink=k, waves=w, loads=l))
                         for b, k in zip(bufs, sinks)]
                ms, clock = timed_calls(calls, args.steps, args.warmup, args.clock_warmup)
                print(json.dumps({"workload": "read_floor", "size": name, "bytes": nb, "copies": cps,
                                  "waves_per_workgroup": waves, "kb_per_wave": loads,
                                  "steps": args.steps, "us": round(ms * 1e3, 3),
                                  "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "kernel": "stream_read_kernel<%d>" % loads}), flush=True)
                del sinks, calls
            del bufs
            torch.cuda.empty_cache()
        return
    if args.workload == "gemm_12288x4096_n4096":
        print(json.dumps(gemm_secondary(args.gemm_iters, args.gemm_warmup)), flush=True)
        return
    if args.workload == "quantize_12288x4096":
        # fp16 weights -> packed codes, scales, packed zeros; 4 copies of the
        # 100 MB input cycled through (400 MB, past the last-level cache)
        M, K = 12288, 4096
        G = K // GROUP
        w0 = torch.from_numpy(inputs.fp16_weights(M, K, wid=6)).cuda()
        ws = [w0] + [w0.clone() for _ in range(3)]
        outs = [B.quantize(w) for w in ws]
        calls = [(lambda w=w, o=o: B.lib().w4a16_quantize(
            w.data_ptr(), M, K, GROUP, o[0].data_ptr(), o[1].data_ptr(), o[2].data_ptr(),
            torch.cuda.current_stream().cuda_stream)) for w, o in zip(ws, outs)]
        stream = torch.cuda.Stream()
        g = capture(calls, stream)
        time_graph(g, 5, stream)
        reps = 50
        ms = time_graph(g, reps, stream) / (reps * len(calls))
        b = 2 * M * K + M * K // 2 + 2 * M * G + M * G // 2
        print(json.dumps({"workload": "quantize_12288x4096", "us": round(ms * 1e3, 3), "bytes_per_call": b,
                          "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "kernel": "quantize_kernel"}), flush=True)
        return
    if args.workload == "decode_step":
        # a LLaMA-7B decode step: 32 decoder layers (QKV, attention, o_proj,
        # gate/up, down, with the normalizations and the gated activation),
        # one HIP graph per step, B sequences at context ~1024 in a 2048-slot
        # cache; embeddings and the output head are not part of it
        from gemm_w4a16_group_amd.decode import DecodeGraph
        H, D, I, S, L = 32, 128, 11008, 2048, 32
        for Bn in (1, 8):
            layers = []
            for layer in range(L):
                ly = {}
                for proj, (name, M, K) in enumerate((("qkv", 3 * H * D, H * D), ("o", H * D, H * D),
                                                     ("gate_up", 2 * I, H * D), ("down", H * D, I))):
                    w = torch.from_numpy(inputs.raw_q_words(M, K, wid=11, layer=layer, proj=proj).view("int32")).cuda()
                    sc, z = inputs.scales_zeros(M, K, wid=11, layer=layer, proj=proj)
                    _, zd = B.pack(None, torch.from_numpy(z).cuda())
                    ly[name] = (w, torch.from_numpy(sc).cuda(), zd)
                _, _, g1 = inputs.hidden_states(1, H * D, wid=11, layer=2 * layer)
                _, _, g2 = inputs.hidden_states(1, H * D, wid=11, layer=2 * layer + 1)
                ly["attn_norm"], ly["mlp_norm"] = torch.from_numpy(g1).cuda(), torch.from_numpy(g2).cuda()
                ly["k_cache"] = torch.randn((Bn, H, S, D), dtype=torch.float16, device="cuda",
                                            generator=torch.Generator(device="cuda").manual_seed(layer))
                ly["v_cache"] = torch.randn((Bn, H, S, D), dtype=torch.float16, device="cuda",
                                            generator=torch.Generator(device="cuda").manual_seed(1000 + layer))
                layers.append(ly)
            pos0 = [1023] * Bn
            dg = DecodeGraph(layers, pos0, max_len=S)
            _, emb, _ = inputs.hidden_states(Bn, H * D, wid=11, layer=99)
            dg.embed.copy_(torch.from_numpy(emb).cuda())   # the same token embedding every step
            dg.step()            # eager (loads the kernels)
            dg.step()            # capture + first replay
            torch.cuda.synchronize()
            steps = 50
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            for _ in range(steps):
                dg.step()
            end.record()
            end.synchronize()
            ms = start.elapsed_time(end) / steps
            wbytes = L * sum(alg_bytes(M, K, Bn) for M, K in ((3 * H * D, H * D), (H * D, H * D), (2 * I, H * D),
                                                             (H * D, I)))
            kv = L * 2 * Bn * H * D * 2 * (1024 + 2 + steps // 2)
            print(json.dumps({"workload": "llama7b_decode_step", "B": Bn, "layers": L, "context": "1025-%d" % (1026 + steps),
                              "ms_per_step": round(ms, 4), "tokens_per_s": round(Bn * 1e3 / ms, 1),
                              "weights_GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
                              "weights_plus_kv_GB/s": round((wbytes + kv) / (ms * 1e-3) / 1e9, 1),
                              "finite": bool(torch.isfinite(dg.hidden()).all().item())}), flush=True)
            del dg, layers
            torch.cuda.empty_cache()
        return
    if args.workload == "tune_table":
        # the tuner's choice per N for the 12288x4096 projection (cold-cache
        # timing inside the tuner), then the tuned and the default plan timed
        # the same way as small_n / large_n (graph of calls over 40 weight
        # copies), both layouts
        M, K = 12288, 4096
        cps = 40
        lay = Layer(M, K, 10, copies=cps)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        for layout in (B.LAYOUT_KN, B.LAYOUT_TOKEN):
            for N in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 4096):
                xh = inputs.activations(K, N, wid=10)
                x = torch.from_numpy(xh.T.copy() if layout == B.LAYOUT_TOKEN else xh).cuda()
                qpk, sd, zpk = lay.copies[0]
                tuned, tuner_us, tried = B.tune(qpk, sd, zpk, x, layout=layout, iters=5, flush=flush)
                shape = (N, M) if layout == B.LAYOUT_TOKEN else (M, N)
                ncalls = cps if N <= 256 else 4
                outs = [torch.empty(shape, dtype=torch.float16, device="cuda") for _ in range(ncalls)]
                res = {}
                for name, plan in (("default", None), ("tuned", tuned)):
                    calls = [(lambda c=c, o=o, pl=plan: B.gemm(c[0], c[1], c[2], x, out=o, plan=pl, layout=layout))
                             for c, o in zip(lay.copies[:ncalls], outs)]
                    stream = torch.cuda.Stream()
                    g = capture(calls, stream)
                    reps = max(2, (args.steps // ncalls) if N <= 256 else 5)
                    warm_graph(g, stream, 0.3)
                    res[name] = time_graph(g, reps, stream) / (reps * ncalls) * 1e3
                    del g
                print(json.dumps({"workload": "tune_table_12288x4096", "layout": "token" if layout else "kn",
                                  "N": N, "plans_timed": tried, "tuner_us": round(tuner_us, 3),
                                  "default_us": round(res["default"], 3), "tuned_us": round(res["tuned"], 3),
                                  "default": B.plan_default(M, N, K, layout).as_dict(),
                                  "tuned": tuned.as_dict()}), flush=True)
        return
    if args.workload == "attention":
        # one decode step of LLaMA-7B attention (32 heads of 128) over a KV
        # cache of capacity S; copies of the caches cycled through so that
        # they are read from HBM
        H, D = 32, 128
        for Bn, S, lens, bound in ((1, 4096, [512], "tight"), (1, 4096, [2048], "tight"),
                                   (1, 4096, [4096], "tight"), (1, 4096, [512], "capacity"),
                                   (8, 2048, [int(v) for v in np.random.default_rng(8).integers(1, 2049, 8)], "tight"),
                                   (32, 1024, [1024] * 32, "tight")):
            pos = np.array(lens, dtype=np.int32) - 1
            max_len = int(pos.max()) + 1 if bound == "tight" else S
            qkv_h, kc_h, vc_h = inputs.attention_inputs(Bn, H, D, S, wid=9)
            rd = 2 * int(pos.sum()) * H * D * 2
            b_alg = rd + Bn * 3 * H * D * 2 + Bn * H * D * 2 + 2 * Bn * H * D * 2
            cps = max(4, int(1.1e9 // max(rd, 1)))
            cps = min(cps, max(4, int(8e9 // (2 * kc_h.nbytes))))
            qkv = torch.from_numpy(qkv_h).cuda()
            pos_d = torch.from_numpy(pos).cuda()
            kcs = [torch.from_numpy(kc_h).cuda() for _ in range(cps)]
            vcs = [torch.from_numpy(vc_h).cuda() for _ in range(cps)]
            outs = [torch.empty((Bn, H * D), dtype=torch.float16, device="cuda") for _ in range(cps)]
            calls = [(lambda k=k, v=v, o=o: B.decode_attention(qkv, k, v, pos_d, max_len=max_len, out=o))
                     for k, v, o in zip(kcs, vcs, outs)]
            stream = torch.cuda.Stream()
            g = capture(calls, stream)
            warm_graph(g, stream, 0.3)
            reps = max(2, args.steps // cps)
            us = time_graph(g, reps, stream) / (reps * cps) * 1e3
            print(json.dumps({"workload": "decode_attention", "B": Bn, "H": H, "D": D, "S": S,
                              "lengths": lens if Bn <= 8 else "%d x %d" % (Bn, lens[0]), "max_len": max_len,
                              "us": round(us, 3), "bytes": b_alg, "GB/s": round(b_alg / (us * 1e-6) / 1e9, 1),
                              "frac_hbm": round(b_alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
            del g, calls, kcs, vcs, outs
            torch.cuda.empty_cache()
        return
    if args.workload == "prologue":
        # residual add + RMS normalization feeding the QKV and gate/up
        # projections (token-major), against the projection alone and the
        # normalization alone; weight copies cycled through as in the GEMV
        for name, M, K in (("qkv", 12288, 4096), ("gate_up", 22016, 4096)):
            cps = max(8, int(1.1e9 // alg_bytes(M, K, 1)))
            lay = Layer(M, K, 7, copies=cps)
            for N in (1, 16, 128):
                xh, rh, gh = inputs.hidden_states(N, K, wid=7)
                x, r, gm = (torch.from_numpy(a).cuda() for a in (xh, rh, gh))
                xs = [x.clone() for _ in range(cps)]
                hs = [torch.empty_like(x) for _ in range(cps)]
                ys = [torch.empty_like(x) for _ in range(cps)]
                outs = [torch.empty((N, M), dtype=torch.float16, device="cuda") for _ in range(cps)]
                variants = {
                    "gemm": [(lambda c=c, o=o, xx=xx: B.gemm(c[0], c[1], c[2], xx, out=o, layout=B.LAYOUT_TOKEN))
                             for c, o, xx in zip(lay.copies, outs, xs)],
                    "add_rmsnorm": [(lambda xx=xx, h=h, y=y: B.add_rmsnorm(xx, r, gm, 1e-6, h=h, y=y))
                                    for xx, h, y in zip(xs, hs, ys)],
                    "fused": [(lambda c=c, o=o, xx=xx, h=h: B.gemm_add_rmsnorm(c[0], c[1], c[2], xx, r, gm, 1e-6,
                                                                             h=h, out=o))
                              for c, o, xx, h in zip(lay.copies, outs, xs, hs)],
                }
                res = {}
                for vname, calls in variants.items():
                    stream = torch.cuda.Stream()
                    g = capture(calls, stream)
                    warm_graph(g, stream, 0.3)
                    reps = max(2, args.steps // cps)
                    res[vname] = time_graph(g, reps, stream) / (reps * cps) * 1e3
                    del g
                nb = 8 * N * K + 2 * K
                print(json.dumps({"workload": "prologue_" + name, "M": M, "K": K, "N": N,
                                  "gemm_us": round(res["gemm"], 3), "add_rmsnorm_us": round(res["add_rmsnorm"], 3),
                                  "fused_us": round(res["fused"], 3),
                                  "fused_over_gemm_us": round(res["fused"] - res["gemm"], 3),
                                  "add_rmsnorm_GB/s": round(nb / (res["add_rmsnorm"] * 1e-6) / 1e9, 1),
                                  "plan": B.plan_default(M, N, K, B.LAYOUT_TOKEN).as_dict()}), flush=True)
            del lay
            torch.cuda.empty_cache()
        return
    if args.workload == "gemv_4096x4096":
        ms, plan, *_ = gemv_rotation(4096, 4096, 1, max(args.copies, 120), args.steps, args.warmup,
                                     clock_s=args.clock_warmup)
        rows.append(("gemv_4096x4096", 4096, 4096, 1, ms, plan))
    elif args.workload == "decode_linears":
        for proj, (name, M, K) in enumerate(inputs.LLAMA7B_PROJ):
            cps = max(8, int(1.1e9 // alg_bytes(M, K, 1)))
            ms, plan, *_ = gemv_rotation(M, K, 2, cps, args.steps, args.warmup, clock_s=args.clock_warmup)
            rows.append((name, M, K, 1, ms, plan))
    elif args.workload in ("small_n", "large_n"):
        Ns = [1, 2, 4, 8, 16, 32] if args.workload == "small_n" else [64, 128, 256, 512, 1024, 2048, 4096]
        wid = 3 if args.workload == "small_n" else 4
        M, K = 12288, 4096
        cps = 40
        lay = Layer(M, K, wid, copies=cps)
        layout = B.LAYOUT_TOKEN if args.token else B.LAYOUT_KN
        for N in Ns:
            xh = inputs.activations(K, N, wid=wid)
            x = torch.from_numpy(xh.T.copy() if args.token else xh).cuda()
            shape = (N, M) if args.token else (M, N)
            outs = [torch.empty(shape, dtype=torch.float16, device="cuda") for _ in range(cps)]
            ncalls = cps if N <= 256 else 4
            calls = [(lambda c=c, o=o: B.gemm(c[0], c[1], c[2], x, out=o, layout=layout))
                     for c, o in zip(lay.copies[:ncalls], outs[:ncalls])]
            stream = torch.cuda.Stream()
            g = capture(calls, stream)
            reps = max(2, (args.steps // ncalls) if N <= 256 else 5)
            warm_graph(g, stream, 0.3)
            ms = time_graph(g, reps, stream) / (reps * ncalls)
            rows.append(("12288x4096" + ("_token" if args.token else ""), M, K, N, ms,
                         B.plan_default(M, N, K, layout).as_dict()))
    elif args.workload == "stack":
        for N in (1, 16):
            mats = []
            for layer in range(32):
                for proj, (name, M, K) in enumerate(inputs.LLAMA7B_PROJ):
                    w = torch.from_numpy(inputs.raw_q_words(M, K, wid=5, layer=layer, proj=proj).view("int32")).cuda()
                    s, z = inputs.scales_zeros(M, K, wid=5, layer=layer, proj=proj)
                    _, zd = B.pack(None, torch.from_numpy(z).cuda())
                    x = torch.from_numpy(inputs.activations(K, N, wid=5, layer=layer, proj=proj)).cuda()
                    o = torch.empty((M, N), dtype=torch.float16, device="cuda")
                    mats.append((w, torch.from_numpy(s).cuda(), zd, x, o))
            calls = [(lambda m=m: B.gemm(m[0], m[1], m[2], m[3], out=m[4])) for m in mats]
            stream = torch.cuda.Stream()
            g = capture(calls, stream)
            time_graph(g, 3, stream)
            reps = 20
            ms = time_graph(g, reps, stream) / reps
            wbytes = sum(alg_bytes(M, K, N) for (_, M, K) in inputs.LLAMA7B_PROJ) * 32
            print(json.dumps({"workload": "llama7b_stack_32x4", "N": N, "ms_per_step": round(ms, 4),
                              "steps_per_s": round(1e3 / ms, 1),
                              "GB/s": round(wbytes / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
            del mats, calls, g
            torch.cuda.empty_cache()
        return
    for (name, M, K, N, ms, plan) in rows:
        b = alg_bytes(M, K, N)
        f = alg_flops(M, K, N)
        print(json.dumps({"workload": name, "M": M, "K": K, "N": N, "us": round(ms * 1e3, 3),
                          "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "TFLOP/s": round(f / (ms * 1e-3) / 1e12, 2),
                          "frac_mfma": round(f / (ms * 1e-3) / 1e12 / FP16_PEAK_TFLOPS, 4),
                          "plan": plan}), flush=True)


def short_kernel_name(name):
    """A profiler's kernel name reduced to the form w4a16_kernel_name prints:
    no return type, namespaces or parameter list ("void ns::(anonymous
    namespace)::tiled_kernel<512, 128, 8, 8, 2, 1>(ns::GemmArgs, int)" ->
    "tiled_kernel<512, 128, 8, 8, 2, 1>")."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not name.startswith("(anonymous", i):
            cut = i
            break
    name = name[:cut]
    depth, start = 0, 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and name[i:i + 2] == "::":
            start = i + 2
    return name[start:].strip()


def kernel_matches(name, query):
    """Profiler kernel name against a query: the short name exactly, or a
    substring of the full name when the query starts with "~"."""
    if query.startswith("~"):
        return query[1:] in name
    return short_kernel_name(name) == query


def trace_summary(path, kernel, last):
    """Durations of the last ``last`` dispatches of ``kernel`` in a rocprofv3
    kernel trace (csv), i.e. the timed calls of a bench run; no GPU."""
    import csv
    import glob
    import statistics
    files = [path] if os.path.isfile(path) else sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"),
                                                                 recursive=True))
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_matches(r.get("Kernel_Name", ""), kernel):
                    rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    if last > 0:
        rows = rows[-last:]
    if not rows:
        print(json.dumps({"kernel": kernel, "dispatches": 0}))
        return
    d = [(e - b) / 1e3 for b, e in rows]
    span = (rows[-1][1] - rows[0][0]) / 1e3
    print(json.dumps({"kernel": kernel, "dispatches": len(d), "median_us": round(statistics.median(d), 3),
                      "mean_us": round(statistics.fmean(d), 3), "min_us": round(min(d), 3),
                      "max_us": round(max(d), 3), "span_us_per_dispatch": round(span / len(d), 3),
                      "files": files}))


XCDS = 8   # accelerator complex dies of an MI355X


def counter_summary(path, kernel):
    """Means per dispatch of the rocprofv3 --pmc counters recorded for
    ``kernel`` (csv files under ``path``), with the derived ratios they
    allow, over the per-XCD cycle count (GRBM_GUI_ACTIVE counts the eight
    XCDs together, so one XCD's cycles are an eighth of it): MFMA busy
    (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs), VALU and LDS issue busy
    (SQ_ACTIVE_INST_* over 256 CUs), TA / TD busy (summed over 256 CUs),
    the clock those cycles imply over the kernel's traced duration when
    given, mean waves resident per CU (SQ_WAVE_CYCLES / SQ_BUSY_CYCLES),
    instruction mix per wave; no GPU.  Short kernels read high (the
    counters run a little past the kernel)."""
    import collections
    import csv
    import glob
    files = [path] if os.path.isfile(path) else sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                                                 recursive=True))
    acc = collections.defaultdict(list)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel_matches(r.get("Kernel_Name", ""), kernel):
                    acc[r["Counter_Name"]].append(float(r["Counter_Value"]))
    c = {k: sum(v) / len(v) for k, v in acc.items()}
    out = {"kernel": kernel, "dispatches": max((len(v) for v in acc.values()), default=0),
           "counters": {k: round(v, 1) for k, v in sorted(c.items())}}
    g = c.get("GRBM_GUI_ACTIVE")
    if g:
        g = g / XCDS
        out["xcd_cycles"] = round(g, 1)
        for k, name, units in (("SQ_VALU_MFMA_BUSY_CYCLES", "mfma_busy", 1024),
                               ("SQ_ACTIVE_INST_VALU", "valu_busy", 256), ("SQ_ACTIVE_INST_LDS", "lds_busy", 256),
                               ("TA_TA_BUSY_sum", "ta_busy", 256), ("TD_TD_BUSY_sum", "td_busy", 256)):
            if k in c:
                out[name] = round(c[k] / (units * g), 4)
    if c.get("SQ_BUSY_CYCLES") and "SQ_WAVE_CYCLES" in c:
        out["waves_per_busy_cycle"] = round(c["SQ_WAVE_CYCLES"] / c["SQ_BUSY_CYCLES"], 3)
    if c.get("SQ_WAVES"):
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU"):
            if k in c:
                out["per_wave_" + k[9:].lower()] = round(c[k] / c["SQ_WAVES"], 1)
    print(json.dumps(out))


# (tag, kernel as w4a16_kernel_name prints it, M, K, N, bench.py arguments) of
# the HBM-traffic records; "readcal" (the read probe over 512 MiB) calibrates
# the read counters, "copy" (a torch copy of 512 MiB) the write counter
TRAFFIC_RUNS = [
    ("readcal", "stream_read_kernel<4>", 0, 0, 0, "--workload read_calib"),
    ("copy", "~elementwise_kernel", 0, 0, 0, "--workload copy_calib"),
    ("gemv", "skinny_kernel<1, 4>", 12288, 4096, 1, "--steps 400 --warmup 40 --no-gemm --no-cpu-baseline"),
    ("gemm", "tiled_dx_kernel<512, 128, 8, 8, 2, 1>", 12288, 4096, 4096,
     "--workload gemm_12288x4096_n4096 --gemm-iters 5 --gemm-warmup 3"),
]


def traffic_commands(tag, args_):
    return ["rocprofv3 --pmc %s -d /tmp/prof_%s_%s -o pmc --output-format csv -- python3 bench.py %s"
            % (ctr, tag, name, args_) for ctr, name in (("FETCH_SIZE", "READ"), ("WRITE_SIZE", "WRITE"))]


def write_traffic(path):
    """profiles/traffic_counters.{json,md} from the per-run counter summaries
    <tag>_READ.json and <tag>_WRITE.json under ``path`` (each the output of
    --counter-summary for TRAFFIC_RUNS' kernel); no GPU."""
    def counters(tag, part, kernel):
        with open(os.path.join(path, "%s_%s.json" % (tag, part))) as fh:
            for line in fh:
                d = json.loads(line)
                if d["kernel"] == kernel:
                    return d["counters"], d["dispatches"]
        raise KeyError("%s %s %s" % (tag, part, kernel))
    nb = 512 << 20
    rc, _ = counters("readcal", "READ", TRAFFIC_RUNS[0][1])
    wc, _ = counters("copy", "WRITE", TRAFFIC_RUNS[1][1])
    cal = {"read_kernel": "the streaming-read probe (stream_read_kernel<4>) over 512 MiB",
           "write_kernel": "torch fp16 elementwise copy (torch.mul(src, 1, out=dst)), 256 Mi elements",
           "bytes_read": nb, "bytes_written": nb, "fetch_kib": round(rc["FETCH_SIZE"], 1),
           "write_kib": round(wc["WRITE_SIZE"], 1), "fetch_factor": nb / (rc["FETCH_SIZE"] * 1024),
           "write_factor": nb / (wc["WRITE_SIZE"] * 1024),
           "commands": traffic_commands("readcal", TRAFFIC_RUNS[0][5])[:1] + traffic_commands("copy", TRAFFIC_RUNS[1][5])[1:]}
    recs = {}
    lines = ["HBM traffic per launch from rocprofv3 counters, one MI355X", "",
             "Calibration: %s reads %d B per launch; FETCH_SIZE reads %.1f KiB (fetch_factor %.5f)."
             % (cal["read_kernel"], nb, cal["fetch_kib"], cal["fetch_factor"]),
             "%s writes %d B; WRITE_SIZE reads %.1f KiB (write_factor %.5f)."
             % (cal["write_kernel"], nb, cal["write_kib"], cal["write_factor"])]
    lines += ["  " + c for c in cal["commands"]] + [""]
    for tag, kern, M, K, N, a in TRAFFIC_RUNS[2:]:
        r_, nf = counters(tag, "READ", kern)
        w_, _ = counters(tag, "WRITE", kern)
        f, w = r_["FETCH_SIZE"], w_["WRITE_SIZE"]
        b = f * 1024 * cal["fetch_factor"] + w * 1024 * cal["write_factor"]
        r = {"fetch_kib": round(f, 1), "write_kib": round(w, 1), "dispatches": nf,
             "sources_sha256": sources_sha(kern), "bytes_per_launch": int(round(b)),
             "algorithmic_bytes": alg_bytes(M, K, N), "commands": traffic_commands(tag, a)}
        recs["%s@%dx%dx%d" % (kern, M, K, N)] = r
        lines.append("%s@%dx%dx%d: FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB per dispatch (mean of %d dispatches)"
                     % (kern, M, K, N, f, w, nf))
        lines.append("  HBM bytes per launch %d = %.3f x the algorithmic %d"
                     % (r["bytes_per_launch"], b / r["algorithmic_bytes"], r["algorithmic_bytes"]))
        lines += ["  " + c for c in r["commands"]] + [""]
    lines.append("Summaries: python3 bench.py --counter-summary /tmp/prof_<tag>_<READ|WRITE> --kernel <kernel> "
                 "> <tag>_<READ|WRITE>.json;")
    lines.append("this file: python3 bench.py --write-traffic <directory of those summaries>.")
    out = {"note": "HBM bytes per launch = FETCH_SIZE KiB * 1024 * fetch_factor + WRITE_SIZE KiB * 1024 * "
                   "write_factor; the factors make the counters read the calibration kernels' known bytes. Counters "
                   "were taken on the sources whose sha256 is stored; bench.py reports null traffic once they change.",
           "calibration": cal, "kernels": recs}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", "traffic_counters.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.kernel, args.last)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.kernel)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from gemm_w4a16_group_amd import binding
    binding.load_library()
    if args.workload == "gemv_12288x4096":
        headline(args)
    else:
        extra(args)


if __name__ == "__main__":
    main()
