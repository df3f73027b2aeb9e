#!/usr/bin/env python3
"""Benchmark of the NVFP4 routed-expert MoE layer on one MI355X.

Headline (`value`): prefill tokens/s of one MoE layer at 8192 tokens (top-8 Zipf(1.1)
routing over 512 experts, hidden 2048, expert intermediate 768, bf16 in and out); a
step is one nvfp4_moe_prefill call (route, activation staging, gate/up + SwiGLU, down +
weighted combine, final rounding). Steps rotate over 48 distinct device copies of the
layer (65 GB), so no step finds its weights in the 256 MB Infinity Cache.

Also reported on the same line: per-kernel times from HIP events on the launch stream
and the roofline of the dominant kernel (the gate/up grouped GEMM against the dense
fp16 matrix-core peak), decode HBM bandwidth at 1 and 4 tokens (hipGraph of 48
layer calls, replayed), the W4A8 and W4A4 prefills at 32768 tokens, the router, the Q8_0-down
layer, the host-CPU decode projection, and the CPU oracle timed on a bounded sample of
the prefill workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak
PEAK_INT8_TOPS = 5000.0
PEAK_HBM_GBS = 8000.0
N_LAYERS = 48
GATEUP_BYTES = 2 * 768 * 2048 * 9 // 16      # NVFP4 gate + up of one expert (codes + scales)
DOWN_BYTES_NVFP4 = 2048 * 768 * 9 // 16      # NVFP4 down
DOWN_BYTES_Q8 = 2048 * 768 + 2048 * 24 * 2   # Q8_0 down: int8 codes + fp16 scales per 32 inputs


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=N_LAYERS)
    ap.add_argument("--decode-rounds", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=512)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "w4a8", "w4a4", "q8down", "router", "host",
                                       "shared"],
                    default="all")
    ap.add_argument("--decode-tokens", type=int, choices=[0, 1, 4], default=0,
                    help="decode leg: only the 1-token or only the 4-token workload (0: both)")
    ap.add_argument("--w4a8-variant", choices=["both", "f16", "int8"], default="both",
                    help="W4A8 leg: fp16 matrix cores, int8 matrix cores, or both")
    ap.add_argument("--eager", action="store_true",
                    help="time the prefill steps and the decode calls as plain launch loops instead of "
                         "hipGraph replays (for counter runs)")
    ap.add_argument("--no-stage-times", action="store_true",
                    help="skip the per-stage event pass, so a kernel trace of the run holds the timed steps "
                         "(and the warm-up before them) only")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print a markdown table of a rocprofv3 kernel trace: per kernel, the last --take "
                         "dispatches (the timed steps) and nothing else runs")
    ap.add_argument("--take", type=int, default=0, help="dispatches per kernel kept by --summarize-trace")
    ap.add_argument("--match", default="nvfp4::",
                    help="--summarize-trace keeps kernels whose name contains this (default: the library's)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run device-to-device copies of 1 GiB (the plain copy kernel whose HBM "
                         "counter readings scale the GEMM's FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def replicate(layer, n):
    """n distinct device copies of one layer (same bytes, different addresses)."""
    import nvfp4_quantized_moe_02_amd as nv
    out = [layer]
    for _ in range(n - 1):
        out.append(nv.Layer(*[type(p)(p.codes.clone(), p.scales.clone(),
                                      None if p.gamma is None else p.gamma.clone())
                              for p in (layer.gate, layer.up, layer.down)]))
    return out


def stage_times(calls, steps, nstages):
    """Mean ms per launch of each stage: stage s of `steps` calls (rotating over the layer
    copies) captured back to back in a hipGraph, replayed once untimed and once between two
    events on the launch stream (the decode legs time their stages the same way). Every
    call shares the workspace, activations and routing, so after one full call stage s of
    any call finds its inputs there. An event pair around each eager staged call would also
    time the host's launch latency and the events' own synchronisation between kernels."""
    import torch
    out = []
    calls[0].run()  # every stage's inputs in the workspace
    for s in range(nstages):
        torch.cuda.synchronize()
        st = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for i in range(steps):
                calls[i % len(calls)].stage(s)
        g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        out.append(t0.elapsed_time(t1) / steps)
        del g
    return out


def timed_steps(calls, steps, warmup):
    """ms per step: `warmup` eager calls, then the `steps` calls (rotating over the layer
    copies) captured once in a hipGraph; one untimed replay, then one timed replay."""
    import torch
    for i in range(warmup):
        calls[i % len(calls)].run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            calls[i % len(calls)].run()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del g
    return ms


def eager_steps(calls, steps):
    """ms per step of the same calls as a plain launch loop (no graph)."""
    import torch
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        calls[i % len(calls)].run()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def bench_prefill(layers, index, act, steps, warmup, stage_pass=True, eager=False, shared=None):
    """shared: per-layer shared experts (one-expert layers, same count as layers), or None.
    The shared-expert call has no staged form: no stage pass with it."""
    import numpy as np
    import torch
    import nvfp4_quantized_moe_02_amd as nv
    import workloads as W
    wl = W.draw_workload(index)
    dev = "cuda"
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.from_numpy(wl.ids).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    L0 = layers[0]
    out = torch.empty((wl.T, L0.H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(nv.prefill_workspace_size(wl.T, L0.H, L0.I, L0.E, 8, act, shared=shared is not None),
                     dtype=torch.uint8, device=dev)
    calls = [nv.PreparedCall("prefill", x, L, ids, w, out, ws, act=act,
                             shared=None if shared is None else shared[i]) for i, L in enumerate(layers)]
    stage_pass = stage_pass and shared is None
    if eager:
        for i in range(warmup):
            calls[i % len(calls)].run()
        ms = eager_steps(calls, steps)
    else:
        ms = timed_steps(calls, steps, warmup)
    if stage_pass:
        # the eager loop first: the stage pass's timed launches are then the last of each
        # kernel in a trace of this run (so a summary of the last `steps` dispatches per
        # kernel holds exactly the launches whose event time this reports)
        ms_eager = eager_steps(calls, steps)
        st = stage_times(calls, steps, 4)
    else:
        st, ms_eager = [float("nan")] * 4, float("nan")
    P = wl.T * 8
    H, I = L0.H, L0.I
    if shared is not None:
        P += wl.T  # the shared expert's pairs
    gu_flops = 2.0 * P * (2 * I) * H
    dn_flops = 2.0 * P * H * I
    counts = np.bincount(wl.ids.reshape(-1), minlength=L0.E)
    tiles = int(np.sum((counts + 127) // 128))
    return dict(T=wl.T, ms=ms, ms_eager=ms_eager, stages_ms=st, gu_flops=gu_flops, dn_flops=dn_flops,
                padded_frac=P / (tiles * 128.0), tokens_per_s=wl.T / (ms / 1e3))


def bench_decode(layers, index, rounds, down_bytes=DOWN_BYTES_NVFP4, eager=False, shared=None):
    """hipGraph of one call per layer (48 layers), replayed `rounds` times (eager: the same
    calls as a plain launch loop, for counter runs). down_bytes: bytes of one expert's down
    projection (NVFP4 or Q8_0)."""
    import numpy as np
    import torch
    import nvfp4_quantized_moe_02_amd as nv
    import workloads as W
    wl = W.draw_workload(index)
    dev = "cuda"
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(dev)
    ids = torch.from_numpy(wl.ids).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    L0 = layers[0]
    out = torch.empty((wl.T, L0.H), dtype=torch.float32, device=dev)
    ws = torch.zeros(nv.decode_workspace_size(wl.T, L0.H, L0.I, L0.E, 8, shared=shared is not None),
                     dtype=torch.uint8, device=dev)
    calls = [nv.PreparedCall("decode", x, L, ids, w, out, ws, shared=None if shared is None else shared[i])
             for i, L in enumerate(layers)]
    res = {}
    legs = (("call", lambda c: c.run()), ("gateup", lambda c: c.stage(0)), ("down", lambda c: c.stage(1)))
    if shared is not None:
        legs = legs[:1]
        res["gateup"] = res["down"] = float("nan")
    for name, fn in legs:
        for c in calls[:4]:
            fn(c)
        torch.cuda.synchronize()
        if eager:
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(rounds):
                for c in calls:
                    fn(c)
            t1.record()
            torch.cuda.synchronize()
            res[name] = t0.elapsed_time(t1) * 1e3 / (rounds * len(calls))
            continue
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                fn(c)
        g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(rounds):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        res[name] = t0.elapsed_time(t1) * 1e3 / (rounds * len(calls))  # us per launch
        del g
    U = len(np.unique(wl.ids)) + (shared is not None)
    byt = U * (GATEUP_BYTES + down_bytes)
    return dict(T=wl.T, unique_experts=U, bytes=byt, us=res["call"], us_gateup=res["gateup"],
                us_down=res["down"], gbs=byt / (res["call"] * 1e-6) / 1e9,
                gbs_gateup=U * 2 * 768 * 2048 * 9 / 16 / (res["gateup"] * 1e-6) / 1e9,
                gbs_down=U * down_bytes / (res["down"] * 1e-6) / 1e9)


def bench_router(T, calls=48, rounds=10):
    """Router (logits -> top-8 -> softmax) on bf16 activations of the 8192-token workload's
    first T rows: microseconds per call from a hipGraph of `calls` calls, replayed (the
    eager time of a call at 1 or 4 tokens is mostly host-side argument handling)."""
    import numpy as np
    import torch
    import nvfp4_quantized_moe_02_amd as nv
    import workloads as W
    x = torch.from_numpy(W.draw_activations(W.config_seed(3), T).view(np.int16)).view(torch.bfloat16).cuda()
    wr = torch.from_numpy(W.draw_router(W.config_seed(3)).view(np.int16)).cuda()
    ws = torch.zeros(nv.router_workspace_size(T, 512), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        nv.router_topk(x, wr, 8, ws=ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(calls):
            nv.router_topk(x, wr, 8, ws=ws)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(rounds):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (rounds * calls)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_host(reps=24):
    """The host-CPU expert projection (nvfp4_moe_decode_host) on a full 512-expert layer in
    host memory: 8 seeded experts tiled to 512 (content does not change the speed), calls
    rotating over `reps` seeded Zipf routings; GB/s counts the weight bytes of the unique
    experts each call reads."""
    import numpy as np
    import torch
    import nvfp4_quantized_moe_02_amd as nv
    import workloads as W
    E, H, I, k = W.EXPERTS, W.HIDDEN, W.INTER, W.TOPK
    sub = W.draw_layer(W.config_seed(3), E=8, H=H, I=I)
    gam = W.draw_gammas(W.config_seed(3), E)

    def tiled(p, name):
        r = E // 8
        return nv.Proj(torch.from_numpy(np.tile(p.codes, (r, 1, 1))), torch.from_numpy(np.tile(p.scales, (r, 1, 1))),
                       torch.from_numpy(gam[name]))
    L = nv.Layer(tiled(sub.gate, "gate"), tiled(sub.up, "up"), tiled(sub.down, "down"))
    per_expert = GATEUP_BYTES + DOWN_BYTES_NVFP4
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    out = {"cpu": cpu_model(), "isa": nv.host_isa(), "threads": threads,
           "workload": "decode projection of one layer on the host CPU (512 NVFP4 experts in host memory, "
                       "top-8 Zipf(1.1) routing, hidden 2048, intermediate 768, FP32 arithmetic)"}
    for T, nt in ((1, threads), (4, threads), (1, 1)):
        calls = []
        for r in range(reps):
            ids = W.draw_routing_zipf(1000 + r, T, E, k)
            calls.append((torch.from_numpy(W.draw_activations(1000 + r, T, H).view(np.int16)).view(torch.bfloat16),
                          torch.from_numpy(ids), torch.from_numpy(W.draw_router_weights(1000 + r, T, k)),
                          len(np.unique(ids))))
        # arguments marshalled once per routing (the C ABI call alone is timed)
        out_t = torch.empty((T, H), dtype=torch.float32)
        prepared = [nv.PreparedHostCall(c[0], L, c[1], c[2], out_t, n_threads=nt) for c in calls]
        for p in prepared[:3]:
            p.run()
        n = reps if nt > 1 else 6
        t = time.perf_counter()
        for p in prepared[:n]:
            p.run()
        dt = (time.perf_counter() - t) / n
        u = sum(c[3] for c in calls[:n]) / n
        out[f"t{T}" + ("_1thread" if nt == 1 else "")] = {"ms": round(dt * 1e3, 3), "unique_experts": round(u, 2),
                                                           "GB/s": round(u * per_expert / dt / 1e9, 1)}
    # then the host's plain streaming read rate on as many threads (torch's multithreaded sum
    # of 2 GiB of float32; measured last, as torch's idle workers spin for a while): the
    # ceiling the projection's byte rate is compared with
    buf = torch.ones(1 << 29, dtype=torch.float32)
    nt0 = torch.get_num_threads()
    torch.set_num_threads(threads)
    buf.sum()
    t = time.perf_counter()
    for _ in range(3):
        buf.sum()
    read_gbs = buf.numel() * 4 * 3 / (time.perf_counter() - t) / 1e9
    torch.set_num_threads(nt0)
    del buf
    out["read_GB/s"] = round(read_gbs, 1)
    for key in ("t1", "t4", "t1_1thread"):
        out[key]["frac_of_read"] = round(out[key]["GB/s"] / read_gbs, 3)
    return out


# Kernel sources whose hash a traffic profile records: counters taken on other sources
# no longer describe the kernel and are not reported.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "prefill_decode_hbm_traffic.md")
TRAFFIC_SOURCES = ["nvfp4_quantized_moe_02_amd/csrc/prefill.hip", "nvfp4_quantized_moe_02_amd/csrc/common.h",
                   "nvfp4_quantized_moe_02_amd/csrc/kernels.h"]


def source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gemm_traffic():
    """HBM bytes per gate/up launch from the committed counter profile, or None when the
    profile is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if line.startswith("traffic-record: "):
                    rec = json.loads(line[len("traffic-record: "):])
                    if rec.get("source_hash") == source_hash():
                        return rec
    except OSError:
        pass
    return None


def copy_calibration():
    """Device-to-device copies of exactly 1 GiB each (read 1 GiB, write 1 GiB)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 4, "source_hash": source_hash()}), flush=True)


def summarize_trace(path, take, match):
    """Markdown table of a rocprofv3 kernel trace (`*_kernel_trace.csv`): for each kernel
    name containing `match`, the last `take` dispatches in start order (all of them when
    take is 0), with their average, minimum and maximum duration in microseconds."""
    import csv
    rows = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if match not in r["Kernel_Name"]:
                continue
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            rows.setdefault(r["Kernel_Name"], []).append((t0, t1))
    out = []
    for name, d in rows.items():
        d.sort()
        kept = d[-take:] if take else d
        us = [(b - a) / 1e3 for a, b in kept]
        out.append((sum(us), name, len(d), len(kept), sum(us) / len(us), min(us), max(us)))
    out.sort(reverse=True)
    tot = sum(o[0] for o in out)
    if not out:
        return
    print("| kernel | dispatches in trace | kept | avg us | min us | max us | % of kept time |")
    print("|---|---|---|---|---|---|---|")
    for t, name, n, k, avg, lo, hi in out:
        print(f"| `{name}` | {n} | {k} | {avg:.2f} | {lo:.2f} | {hi:.2f} | {100 * t / tot:.1f} |")


def cpu_description():
    """The host CPU's model (lscpu's "Model name"), the CPUs it reports (nproc) and the
    CPUs this process may run on."""
    import subprocess
    model = None
    try:
        for line in subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout.splitlines():
            if line.strip().startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True, timeout=10).stdout.strip())
    except (OSError, subprocess.SubprocessError, ValueError):
        nproc = None
    return {"lscpu_model": model or cpu_model(), "nproc": nproc, "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(n_tokens):
    """The float64 oracle on bounded samples: the 8192-token bf16 prefill workload on all
    BLAS threads (the reported value) and on one thread, and the 32768-token W4A8 and W4A4
    workloads on all threads."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle as O
    import workloads as W
    lay = W.draw_layer(W.config_seed(3))
    wl = W.draw_workload(3)
    x = O.bf16_to_f64(wl.x)

    def run(fn, n):
        t = time.perf_counter()
        fn(np.arange(n))
        return time.perf_counter() - t

    dt = run(lambda rows: O.moe_grouped(x, lay, wl.ids, wl.w, rows=rows), n_tokens)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    n1 = max(16, n_tokens // 8)
    with threadpool_limits(limits=1):
        dt1 = run(lambda rows: O.moe_grouped(x, lay, wl.ids, wl.w, rows=rows), n1)
    w4 = W.draw_workload(4)
    n4 = max(16, n_tokens // 2)
    dt4 = run(lambda rows: O.moe_w4a8(w4.x, lay, w4.ids, w4.w, rows=rows), n4)
    n44 = max(16, n_tokens // 4)
    dt44 = run(lambda rows: O.moe_w4a4(w4.x, lay, w4.ids, w4.w, rows=rows), n44)
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n_tokens} tokens of the 8192-token prefill workload (all "
                      f"{len(np.unique(wl.ids[:n_tokens]))} experts they route to), float64 numpy oracle, "
                      f"{dt:.1f} s on {threads} BLAS threads",
            "one_core": {"value": round(n1 / dt1, 3), "unit": "tokens/s", "cores": 1,
                         "sample": f"first {n1} tokens of the same workload, one BLAS thread, {dt1:.1f} s"},
            "w4a8_t32768": {"value": round(n4 / dt4, 3), "unit": "tokens/s", "cores": threads,
                            "sample": f"first {n4} tokens of the 32768-token W4A8 workload (int8 x and h per "
                                      f"row, float64 oracle), {dt4:.1f} s"},
            "w4a4_t32768": {"value": round(n44 / dt44, 3), "unit": "tokens/s", "cores": threads,
                            "sample": f"first {n44} tokens of the same workload with NVFP4 x and h per row "
                                      f"(float64 oracle), {dt44:.1f} s"},
            "host": cpu_description()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.take, args.match)
        return
    import torch
    import nvfp4_quantized_moe_02_amd as nv
    import workloads as W
    nv.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs {props.multi_processor_count}")

    t = time.time()
    lay = W.draw_layer(W.config_seed(3))
    base = nv.Layer.from_numpy(lay, "cuda")
    del lay
    layers = replicate(base, args.layers)
    torch.cuda.synchronize()
    log(f"{args.layers} layers on device in {time.time() - t:.1f} s")

    result = {}
    pre = None
    if args.only in ("all", "prefill"):
        pre = bench_prefill(layers, 3, "bf16", args.steps, args.warmup, not args.no_stage_times, args.eager)
        log(f"prefill 8192: {pre['ms']:.3f} ms/step (graph; eager loop {pre['ms_eager']:.3f}), "
            f"{pre['tokens_per_s']:.0f} tok/s, stages {pre['stages_ms']}")
    dec = {}
    if args.only in ("all", "decode"):
        for idx in (1, 2):
            if args.decode_tokens and W.draw_workload(idx).T != args.decode_tokens:
                continue
            d = bench_decode(layers, idx, args.decode_rounds, eager=args.eager)
            dec[f"t{d['T']}"] = d
            log(f"decode T={d['T']}: {d['us']:.2f} us/layer, {d['gbs']:.0f} GB/s (U={d['unique_experts']}), "
                f"gate/up {d['us_gateup']:.2f} us, down {d['us_down']:.2f} us")
    w4 = w4i = None
    if args.only in ("all", "w4a8"):
        if args.w4a8_variant in ("both", "f16"):
            w4 = bench_prefill(layers, 4, "w4a8_f16", max(4, args.steps // 4), 2, not args.no_stage_times)
            log(f"w4a8 32768: {w4['ms']:.3f} ms/step, {w4['tokens_per_s']:.0f} tok/s, stages {w4['stages_ms']}")
        if args.w4a8_variant in ("both", "int8"):
            w4i = bench_prefill(layers, 4, "w4a8", max(3, args.steps // 8), 1, not args.no_stage_times)
            log(f"w4a8 int8 MFMA 32768: {w4i['ms']:.3f} ms/step, {w4i['tokens_per_s']:.0f} tok/s, "
                f"stages {w4i['stages_ms']}")
    w44 = None
    if args.only in ("all", "w4a4"):
        w44 = bench_prefill(layers, 4, "w4a4", max(4, args.steps // 4), 2, not args.no_stage_times)
        log(f"w4a4 32768: {w44['ms']:.3f} ms/step, {w44['tokens_per_s']:.0f} tok/s, stages {w44['stages_ms']}")
    rt = None
    if args.only in ("all", "router"):
        rt = {f"t{T}_us": round(bench_router(T), 2) for T in (1, 4, 8192)}
        log(f"router: {rt}")
    sh = None
    if args.only in ("all", "shared"):
        # the same layers with a shared expert each (a one-expert layer of the same shape)
        sl = W.draw_shared_expert(W.config_seed(3))
        sbase = nv.Layer.from_numpy(sl, "cuda")
        shared = replicate(sbase, args.layers)
        p = bench_prefill(layers, 3, "bf16", args.steps, args.warmup, shared=shared)
        sh = {"prefill_t8192": {"tokens/s": round(p["tokens_per_s"], 1), "ms_per_step": round(p["ms"], 4),
                                "useful_tflops_step": round((p["gu_flops"] + p["dn_flops"]) / (p["ms"] * 1e-3) / 1e12,
                                                            1)}}
        for idx in (1, 2):
            d = bench_decode(layers, idx, args.decode_rounds, eager=args.eager, shared=shared)
            sh[f"decode_t{d['T']}"] = {"us_per_layer": round(d["us"], 3), "GB/s": round(d["gbs"], 1),
                                       "frac_hbm_peak": round(d["gbs"] / PEAK_HBM_GBS, 4),
                                       "experts_read": d["unique_experts"], "weight_bytes": d["bytes"]}
        log(f"shared expert: {sh}")
        del shared, sbase
    hd = None
    if args.only in ("all", "host"):
        hd = bench_host()
        log(f"host decode: {hd}")
    q8 = None
    if args.only in ("all", "q8down"):
        # the mixed pack's layers: NVFP4 gate/up with a Q8_0 down projection
        del layers, base
        torch.cuda.empty_cache()
        t = time.time()
        lay = W.draw_layer(W.config_seed(3), down_fmt="q8_0")
        base = nv.Layer.from_numpy(lay, "cuda")
        del lay
        layers = replicate(base, args.layers)
        torch.cuda.synchronize()
        log(f"{args.layers} Q8_0-down layers on device in {time.time() - t:.1f} s")
        q8 = {"prefill": bench_prefill(layers, 3, "bf16", max(8, args.steps // 2), args.warmup)}
        for idx in (1, 2):
            d = bench_decode(layers, idx, args.decode_rounds, DOWN_BYTES_Q8)
            q8[f"decode_t{d['T']}"] = d
        log(f"q8 down: prefill {q8['prefill']['ms']:.3f} ms/step, decode T=1 {q8['decode_t1']['us']:.2f} us, "
            f"T=4 {q8['decode_t4']['us']:.2f} us")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_sample_tokens)
        log(f"cpu oracle: {cpu}")

    if pre is not None and not args.no_stage_times:
        gu_ms = pre["stages_ms"][1]
        dn_ms = pre["stages_ms"][2]
        achieved = pre["gu_flops"] / (gu_ms * 1e-3) / 1e12
        trec = gemm_traffic()
        result = {
            "metric": "NVFP4 MoE layer: prefill tokens/s (% MFMA peak); decode HBM GB/s (% peak)",
            "value": round(pre["tokens_per_s"], 1),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(pre["ms"], 4),
            "ms_per_step_eager_loop": round(pre["ms_eager"], 4),
            "timing": ("plain launch loop" if args.eager else
                       "steps captured in one hipGraph and replayed once (after one untimed replay); "
                       "ms_per_step_eager_loop: the same calls as a plain launch loop"),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f16",
            "data": "synthetic: seeded NVFP4 layer (512 experts, H=2048, I=768) copied to 48 device layers; "
                    "seeded bf16 activations and Zipf(1.1) top-8 routing",
            "config": {"workload": "prefill_t8192_zipf: one MoE layer, 8192 tokens, top-8 Zipf(1.1) over 512 "
                                   "experts, hidden 2048, intermediate 768, NVFP4 gate/up/down, bf16 in/out, "
                                   "fp16 matrix cores with fp32 accumulation",
                       "tokens": pre["T"], "experts": 512, "topk": 8, "hidden": 2048, "intermediate": 768,
                       "layers_rotated": args.layers},
            "roofline": {"bound": "mfma", "kernel": "moe_gemm_f16_kernel (gate/up + SwiGLU)",
                         "achieved": round(achieved, 1), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                         "traffic": trec["hbm_bytes_per_launch"] if trec else None,
                         "traffic_source": (f"rocprofv3 FETCH_SIZE + WRITE_SIZE per gate/up launch, scaled by "
                                            f"a 1 GiB copy ({os.path.relpath(TRAFFIC_PROFILE, ROOT)})")
                                           if trec else "no counter profile for the current kernel sources"},
            "prefill_detail": {
                "stage_ms": {"route_stage": round(pre["stages_ms"][0], 4), "gateup": round(gu_ms, 4),
                             "down": round(dn_ms, 4), "finalize": round(pre["stages_ms"][3], 4)},
                "down_tflops": round(pre["dn_flops"] / (dn_ms * 1e-3) / 1e12, 1),
                "useful_tflops_step": round((pre["gu_flops"] + pre["dn_flops"]) / (pre["ms"] * 1e-3) / 1e12, 1),
                "frac_of_fp16_peak_step": round((pre["gu_flops"] + pre["dn_flops"]) / (pre["ms"] * 1e-3) / 1e12
                                                / PEAK_FP16_TFLOPS, 4),
                "row_tile_fill": round(pre["padded_frac"], 4),
            },
        }
    if dec:
        result["decode"] = {k: {"us_per_layer": round(v["us"], 3), "GB/s": round(v["gbs"], 1),
                                "frac_hbm_peak": round(v["gbs"] / PEAK_HBM_GBS, 4),
                                "unique_experts": v["unique_experts"], "weight_bytes": v["bytes"],
                                "us_gateup": round(v["us_gateup"], 3), "us_down": round(v["us_down"], 3),
                                "GB/s_gateup": round(v["gbs_gateup"], 1), "GB/s_down": round(v["gbs_down"], 1),
                                "timing": "hipGraph of 48 layer calls, replayed"}
                            for k, v in dec.items()}
    if w4 is not None:
        result["w4a8"] = {"workload": "32768 tokens, int8 activations (x and h per row), fp16 matrix cores",
                          "tokens/s": round(w4["tokens_per_s"], 1), "ms_per_step": round(w4["ms"], 4),
                          "stage_ms": [round(v, 4) for v in w4["stages_ms"]],
                          "frac_of_fp16_peak_step": round((w4["gu_flops"] + w4["dn_flops"]) / (w4["ms"] * 1e-3)
                                                          / 1e12 / PEAK_FP16_TFLOPS, 4),
                          "frac_of_int8_peak_step": round((w4["gu_flops"] + w4["dn_flops"]) / (w4["ms"] * 1e-3)
                                                          / 1e12 / PEAK_INT8_TOPS, 4)}
    if w4i is not None:
        result["w4a8_int8_mfma"] = {
            "workload": "32768 tokens, the same int8 activations on int8 matrix cores (weights as exact int8 "
                        "2*e2m1, fp32 rescale by e4m3/2 per 16-input group: VALU-bound)",
            "tokens/s": round(w4i["tokens_per_s"], 1), "ms_per_step": round(w4i["ms"], 4),
            "stage_ms": [round(v, 4) for v in w4i["stages_ms"]],
            "frac_of_int8_peak_step": round((w4i["gu_flops"] + w4i["dn_flops"]) / (w4i["ms"] * 1e-3) / 1e12
                                            / PEAK_INT8_TOPS, 4),
            "frac_of_fp16_peak_step": round((w4i["gu_flops"] + w4i["dn_flops"]) / (w4i["ms"] * 1e-3) / 1e12
                                            / PEAK_FP16_TFLOPS, 4)}
    if w44 is not None:
        result["w4a4"] = {"workload": "32768 tokens, NVFP4 activations (x and h per row: E2M1 codes, E4M3 scale "
                                      "per 16, fp32 row scale), fp16 matrix cores",
                          "tokens/s": round(w44["tokens_per_s"], 1), "ms_per_step": round(w44["ms"], 4),
                          "stage_ms": [round(v, 4) for v in w44["stages_ms"]],
                          "frac_of_fp16_peak_step": round((w44["gu_flops"] + w44["dn_flops"]) / (w44["ms"] * 1e-3)
                                                          / 1e12 / PEAK_FP16_TFLOPS, 4)}
    if rt is not None:
        result["router"] = {"workload": "logits of 512 experts (bf16 router matrix, hidden 2048) on bf16 activations, "
                                        "top-8, softmax over the selected logits; us per call in a hipGraph of 48 "
                                        "calls, replayed",
                            **rt}
    if q8 is not None:
        pq = q8["prefill"]
        result["q8_down"] = {
            "workload": "the same layer shape with a Q8_0 down projection (int8 weights, fp16 scale per 32 "
                        "inputs); NVFP4 gate/up",
            "prefill_t8192": {"tokens/s": round(pq["tokens_per_s"], 1), "ms_per_step": round(pq["ms"], 4),
                              "stage_ms": [round(v, 4) for v in pq["stages_ms"]]},
            **{k: {"us_per_layer": round(v["us"], 3), "GB/s": round(v["gbs"], 1),
                   "frac_hbm_peak": round(v["gbs"] / PEAK_HBM_GBS, 4), "weight_bytes": v["bytes"],
                   "us_down": round(v["us_down"], 3), "GB/s_down": round(v["gbs_down"], 1)}
               for k, v in q8.items() if k.startswith("decode")},
        }
        if dec:
            result["q8_down"]["decode_time_vs_nvfp4"] = {
                k: round(q8[f"decode_{k}"]["us"] / dec[k]["us"], 3) for k in dec if f"decode_{k}" in q8}
    if sh is not None:
        result["shared_expert"] = {
            "workload": "the same layers with a shared expert each (an NVFP4 SwiGLU expert of the routed "
                        "experts' shape applied to every token with weight 1, in the same launches); prefill "
                        "8192 tokens, decode 1 and 4 tokens",
            **sh}
    if hd is not None:
        result["host_decode"] = hd
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
