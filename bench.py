#!/usr/bin/env python3
"""Throughput of the routed MoE FFN layer on one MI355X.

One step = one pass of the whole layer (route, bucket, gate/up + SwiGLU, down, combine)
over every layer of the workload, on synthetic seeded inputs already resident in HBM.
The default workload is the GPT-OSS-20B-shaped decode: T = 1 token through 24 independent
layers (H = I = 2880, E = 32, top-4, MXFP4 experts in a 32-slot pool behind a permuted slot
map). Other workloads are selectable with --workload (see synth.CONFIGS).

Output: one JSON line with
  value          MoE-layer tokens/s = T * layers * steps / elapsed (graph replays)
  step_ms        median and p95 of the per-step times (HIP events between replays)
  roofline       the dominant kernel timed with HIP events on its own stream: for decode the
                 fused layer kernel (routing, gate/up, down, combine), priced in algorithmic
                 HBM bytes (the selected experts' code and scale bytes); for prefill the
                 gate/up grouped GEMM, priced in useful MFMA flops (4 * T*k * H * I)
  layer_roofline decode only: selected-expert bytes per layer / graph-replayed layer time
  prefill        the prefill half of the metric (default: the GPT-OSS-20B-shaped prefill,
                 T = 16384): step time, tokens/s, gate/up and down grouped-GEMM MFMA
                 fractions and the per-expert token histogram of the Zipf-biased routing
  cpu_baseline   the fp64 CPU oracle timed on a bounded sample of the headline workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def ggemm_kernel(fmt: str) -> str:
    """The grouped-GEMM kernel that runs a format's prefill expert FFN."""
    return "k_ggemm_mx" if fmt in ("mxfp4", "q6_k") else "k_ggemm"
METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA % of peak"
# bytes per weight of each format: MXFP4 16+1 and Q8_0 32+2 per 32; Q4_K 144, Q5_K 176 and
# Q6_K 210 per 256 (the pool keeps 0.5 more per 32 for Q4_K / Q5_K, the 6-bit scale and min
# in two whole bytes, and 0.25 more for Q6_K, d in a 4-byte record)
BYTES_PER_WEIGHT = {"mxfp4": 17.0 / 32.0, "q8_0": 34.0 / 32.0, "q4_k": 18.0 / 32.0,
                    "q5_k": 22.0 / 32.0, "q6_k": 26.25 / 32.0}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gptoss_decode_t1")
    ap.add_argument("--layers", type=int, default=None, help="override the workload's layer count")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="graph: the step's layer calls are captured once into a HIP graph "
                         "and replayed; eager: every layer call is launched from the host")
    ap.add_argument("--path", choices=("auto", "persistent"), default="auto",
                    help="auto: the library's default launch sequence; persistent: decode "
                         "batches run the layer as one persistent kernel after the router")
    ap.add_argument("--prefill-workload", default="gptoss_prefill",
                    help="prefill workload reported in the line's `prefill` object ('none': skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-oracle baseline sample (0 disables it)")
    ap.add_argument("--stage", action="store_true",
                    help="staged prefill: every third expert is resident, the others are "
                         "copied each step from a backing store into a window of pool slots "
                         "(plan + copy + mapping rewrite before the expert FFN); eager launches")
    ap.add_argument("--stage-overlap", action="store_true",
                    help="with --stage: each layer's plan and copy run on a second stream (default "
                         "priority), one layer ahead, so they overlap the previous layer's "
                         "expert FFN; the compute stream waits on an event before the gate/up")
    return ap.parse_args()


def fused_decode(T, H, E):
    """Whether the library runs the layer as the fused decode kernel (after the router's
    partials): 1 to 4 tokens, T*E <= 256, H <= 4096."""
    return 1 <= T <= 4 and T * E <= 256 and 128 <= H <= 4096


def percentile(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this layer is measured on a single MI355X; multi-GPU sharding is not built.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import quantized_routed_expert_gemv_amd as qm

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = HipEvents()
    cfg = synth.CONFIGS[args.workload]
    res, host_keep = run_workload(cfg, args, args.layers or cfg.layers, args.steps, args.warmup,
                                  hip, qm, synth, np, torch, dev, stage=args.stage)
    result = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": res["config"],
    }
    for key in ("step_ms", "roofline", "layer_roofline", "eager_ms_per_step", "stage_copy",
                "experts"):
        if key in res:
            result[key] = res[key]

    # ---- the prefill half of the metric
    pname = args.prefill_workload
    if pname and pname != "none" and pname != cfg.name and cfg.T <= 16:
        pcfg = synth.CONFIGS[pname]
        torch.cuda.empty_cache()
        psteps = max(3, min(args.steps, 10))
        pres, _ = run_workload(pcfg, args, pcfg.layers, psteps, min(args.warmup, 3), hip, qm, synth,
                               np, torch, dev, keep_host=0)
        pre = {"workload": pcfg.name, "T": pcfg.T, "H": pcfg.H, "I": pcfg.I, "E": pcfg.E,
               "k": pcfg.k, "fmt": pcfg.fmt, "steps": psteps,
               "tokens_per_s": pres["tokens_per_s"], "ms_per_step": pres["ms_per_step"],
               "step_ms": pres["step_ms"], "gate_up": pres["roofline"]}
        for key in ("down", "experts"):
            if key in pres:
                pre[key] = pres[key]
        result["prefill"] = pre

    # ---- CPU baseline: the oracle on a bounded sample of the headline workload
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, host_keep, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def run_workload(cfg, args, n_layers, steps, warmup, hip, qm, synth, np, torch, dev,
                 stage=False, keep_host=4):
    """Time `steps` steps of `cfg` (every layer once per step); returns (figures, host layers
    kept for the CPU baseline)."""
    print(f"[bench] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} "
          f"{cfg.fmt} x {n_layers} layers", file=sys.stderr, flush=True)

    # ---- inputs, resident in HBM before timing
    layers = []
    staged = []             # --stage: (backing store, resident slot map) per layer
    host_keep = []          # a few layers kept on the host for the CPU baseline
    resident = list(range(0, cfg.E, 3))
    window = cfg.E - len(resident)
    for l in range(n_layers):
        L = synth.make_layer(cfg, l)
        if stage:
            by_expert = {n: a[L.slot_map] for n, a in L.planes.items()}
            backing = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I, by_expert, device=dev)
            # resident experts first, then the window (holding stale experts before a copy)
            fill = resident + [(e + 1) % cfg.E for e in range(window)]
            pool = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I,
                                          {n: a[fill] for n, a in by_expert.items()}, device=dev)
            sm_res = np.full(cfg.E, qm.SLOT_MISS, dtype=np.int32)
            sm_res[resident] = np.arange(len(resident), dtype=np.int32)
            staged.append((backing, torch.from_numpy(sm_res).to(dev)))
            del by_expert
        else:
            pool = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I, L.planes, device=dev)
        x = torch.from_numpy(L.x.view(np.int16)).to(dev).view(torch.bfloat16)
        wr = torch.from_numpy(L.wr.view(np.int16)).to(dev).view(torch.bfloat16)
        bias = None if L.bias is None else torch.from_numpy(L.bias).to(dev)
        sm = torch.from_numpy(L.slot_map).to(dev)
        layers.append((pool, x, wr, bias, sm))
        if l < keep_host:
            host_keep.append(L)
        del L
        torch.cuda.synchronize()
    print("[bench] inputs resident", file=sys.stderr, flush=True)

    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    ws = qm.Workspace(T, H, I, E, k, dev)
    outs = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in range(n_layers)]
    stream = torch.cuda.Stream(device=dev)
    prefill = T > 16
    path = qm.PATH_PERSISTENT if args.path == "persistent" else qm.PATH_AUTO
    fused = path == qm.PATH_PERSISTENT and fused_decode(T, H, E)
    # timing events around each layer's dominant launch (recorded by moe_layer_timed on the
    # stream the kernel runs on); created without the system-scope fence that a default
    # event adds on record, which would flush caches between the layer's kernels
    ev = [(hip.create(), hip.create()) for _ in range(n_layers)]
    timed_calls = [qm.LayerCall(pool, sm, wr, bias, x, k, outs[li], ws, path=path,
                                stream=stream, events=ev[li])
                   for li, (pool, x, wr, bias, sm) in enumerate(layers)]
    plain_calls = [qm.LayerCall(pool, sm, wr, bias, x, k, outs[li], ws, path=path,
                                stream=stream)
                   for li, (pool, x, wr, bias, sm) in enumerate(layers)]

    def run(calls):
        for c in calls:
            c()

    copy_ev = []
    mode = args.mode
    if stage:
        if mode == "graph":
            print("[bench] --stage runs eager", file=sys.stderr, flush=True)
            mode = "eager"
        if args.stage_overlap:
            timed_calls, copy_ev = staged_overlap_calls(qm, torch, layers, staged, outs, cfg,
                                                        resident, window, stream, hip, ev)
        else:
            timed_calls, copy_ev = staged_calls(qm, torch, layers, staged, outs, cfg, resident,
                                                window, stream, hip, ev)
        plain_calls = timed_calls

    copy_ms = []

    def eager_pass(n):
        """`n` steps launched from the host, the dominant kernel's events read after each."""
        ms = []
        t0 = time.perf_counter()
        for _ in range(n):
            run(timed_calls)
            stream.synchronize()
            ms.extend(hip.elapsed_ms(a, b) for a, b in ev)
            copy_ms.extend(hip.elapsed_ms(a, b) for a, b in copy_ev)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, ms

    run(plain_calls)                       # load the kernels (and warm caches) once
    stream.synchronize()
    graph = hip.capture(stream.cuda_stream, lambda: run(plain_calls)) if mode == "graph" else None
    for _ in range(warmup):
        if graph is not None:
            hip.launch(graph, stream.cuda_stream)
        else:
            run(timed_calls)
    stream.synchronize()
    torch.cuda.synchronize()

    # ---- timed region: `steps` steps
    step_ev = [hip.create() for _ in range(steps + 1)]
    if graph is not None:
        # the step as it is meant to run: one graph of every layer's launches, replayed; an
        # event between replays gives the per-step times
        t0 = time.perf_counter()
        hip.record(step_ev[0], stream.cuda_stream)
        for i in range(steps):
            hip.launch(graph, stream.cuda_stream)
            hip.record(step_ev[i + 1], stream.cuda_stream)
        stream.synchronize()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        step_ms = [hip.elapsed_ms(step_ev[i], step_ev[i + 1]) for i in range(steps)]
        # ROCm's runtime here refuses event nodes inside a captured graph, so the dominant
        # kernel is timed on an eager pass of the same steps right after
        eager_s, kern_ms = eager_pass(steps)
    else:
        t0 = time.perf_counter()
        eager_s, kern_ms = eager_pass(steps)
        t1 = t0 + eager_s
        step_ms = [eager_s * 1e3 / steps] * steps

    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / steps
    res = {"tokens_per_s": round(T * n_layers * steps / elapsed, 1),
           "ms_per_step": round(ms_per_step, 4),
           "step_ms": {"median": round(percentile(step_ms, 50), 4),
                       "p95": round(percentile(step_ms, 95), 4)},
           "config": {"workload": cfg.name, "T": T, "H": H, "I": I, "E": E, "k": k,
                      "fmt": cfg.fmt, "layers": n_layers, "path": args.path,
                      "launch": ("one HIP graph of the step's moe_layer calls" if mode == "graph"
                                 else "moe_layer per layer, eager")}}
    if graph is not None:
        res["eager_ms_per_step"] = round(eager_s * 1e3 / steps, 4)

    # routing of every layer on the device: distinct experts (decode bytes) and the
    # per-expert token counts (the Zipf load of the prefill workloads)
    n_distinct, counts_all = [], []
    for (pool, x, wr, bias, sm) in layers:
        ids_l, _ = qm.route(x, wr, bias, k)
        ids_np = ids_l.cpu().numpy()
        n_distinct.append(len(np.unique(ids_np)))
        counts_all.append(np.bincount(ids_np.ravel(), minlength=E))

    # ---- roofline of the dominant kernel
    kern_avg_s = float(np.mean(kern_ms)) * 1e-3
    bpw = BYTES_PER_WEIGHT[cfg.fmt]
    if prefill:
        flops = 4.0 * T * k * H * I          # gate and up: 2 flops per weight per pair, twice
        achieved = flops / kern_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": f"gate/up grouped GEMM ({ggemm_kernel(cfg.fmt)})", "work_per_launch": flops}
        c = counts_all[0]
        res["experts"] = {"tokens_per_expert": [int(v) for v in c],
                          "empty": int(np.sum(c == 0)),
                          "under_16": int(np.sum((c > 0) & (c < 16))),
                          "max": int(c.max()), "min_nonempty": int(c[c > 0].min())}
        if not stage:
            res["down"] = time_down_gemm(qm, torch, np, hip, layers[0], cfg, stream, steps)
    else:
        mats = 3 if fused else 2
        bytes_per_launch = float(np.mean(n_distinct)) * mats * I * H * bpw
        achieved = bytes_per_launch / kern_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": ("persistent decode layer: routing, gate/up, down, combine "
                           "(k_gate_up_routed with its down phase)" if fused
                           else "gate/up with the routing finished in-kernel (k_gate_up_routed)"
                           if fused_decode(T, H, E) else "gate/up GEMV (k_gemv)"),
                "work_per_launch": bytes_per_launch}
        layer_bytes = float(np.mean(n_distinct)) * 3 * I * H * bpw
        layer_s = ms_per_step * 1e-3 / n_layers
        res["layer_roofline"] = {
            "bound": "hbm", "achieved": round(layer_bytes / layer_s / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(layer_bytes / layer_s / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_layer": layer_bytes, "us_per_layer": round(layer_s * 1e6, 3),
            "what": "selected-expert code+scale bytes of gate, up and down per layer / "
                    "graph-replayed layer time (router, routing, expert FFN, combine)"}
    roof["traffic"] = measured_traffic(cfg.name)
    roof["avg_launch_us"] = round(kern_avg_s * 1e6, 3)
    roof["method"] = ("HIP events recorded on the kernel's stream around every launch of the "
                      f"dominant kernel in {steps} eager steps ({len(kern_ms)} launches)")
    res["roofline"] = roof
    if stage:
        # the bulk copy: every staged expert's six planes read from the backing store and
        # written into the window (prefill batches use every expert: the whole window)
        per_expert = sum(qm.plane_bytes(cfg.fmt, r, K, sc) for r, K in ((I, H), (I, H), (H, I))
                         for sc in (False, True))
        moved = 2.0 * window * per_expert
        copy_s = float(np.mean(copy_ms)) * 1e-3
        res["config"]["staging"] = {"resident": len(resident), "window": window,
                                    "copy": ("second stream, one layer ahead" if args.stage_overlap
                                             else "in series on the compute stream")}
        res["stage_copy"] = {
            "kernel": "k_stage_copy", "bound": "hbm", "bytes_per_launch": moved,
            "avg_launch_us": round(copy_s * 1e6, 3), "achieved": round(moved / copy_s / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(moved / copy_s / 1e9 / HBM_PEAK_GBS, 4)}
    return res, host_keep


def time_down_gemm(qm, torch, np, hip, layer, cfg, stream, reps):
    """The down grouped GEMM of one prefill layer, alone: route, bucket and gate/up once,
    then `reps` down launches between HIP events on the kernel's stream."""
    pool, x, wr, bias, sm = layer
    T, k, H, I = cfg.T, cfg.k, cfg.H, cfg.I
    with torch.cuda.stream(stream):
        ids, w = qm.route(x, wr, bias, k, stream=stream)
        counts, offsets, perm, inv = qm.bucket(ids, cfg.E, stream=stream)
        h = qm.expert_gate_up(pool, sm, x, k, offsets, perm, stream=stream)
        y = torch.empty((T * k, H), dtype=torch.float32, device=x.device)
        qm.expert_down(pool, sm, T, k, offsets, h, y=y, stream=stream)
        evs = [(hip.create(), hip.create()) for _ in range(reps)]
        for a, b in evs:
            hip.record(a, stream.cuda_stream)
            qm.expert_down(pool, sm, T, k, offsets, h, y=y, stream=stream)
            hip.record(b, stream.cuda_stream)
    stream.synchronize()
    ms = [hip.elapsed_ms(a, b) for a, b in evs]
    flops = 2.0 * T * k * H * I
    s = float(np.mean(ms)) * 1e-3
    return {"bound": "mfma", "achieved": round(flops / s / 1e12, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(flops / s / 1e12 / BF16_PEAK_TFLOPS, 4),
            "kernel": f"down grouped GEMM ({ggemm_kernel(cfg.fmt)})", "work_per_launch": flops,
            "avg_launch_us": round(s * 1e6, 3),
            "method": f"HIP events around {reps} stand-alone launches on the kernel's stream"}


def staged_calls(qm, torch, layers, staged, outs, cfg, resident, window, stream, hip, ev):
    """Per layer: route, bucket, window plan (mapping rewrite), bulk copy of the planned
    experts, gate/up (timed), down, combine -- each a C-ABI stage call on `stream`, with
    every buffer allocated once here."""
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    dev = outs[0].device
    i32 = dict(dtype=torch.int32, device=dev)
    ids = torch.empty((T, k), **i32)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, inv = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    rs = qm._scratch(qm.route_scratch_bytes(T, H, E), dev)
    bs = qm._scratch(qm.bucket_scratch_bytes(T, k, E), dev)
    sm2, cl, cnt = torch.empty(E, **i32), torch.empty(E, **i32), torch.empty(2, **i32)
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    copy_ev = [(hip.create(), hip.create()) for _ in layers]
    first = len(resident)
    calls = []
    for li, (pool, x, wr, bias, _) in enumerate(layers):
        backing, sm_res = staged[li]

        def call(pool=pool, x=x, wr=wr, bias=bias, backing=backing, sm_res=sm_res, li=li):
            qm.route(x, wr, bias, k, ids=ids, w=w, scratch=rs, stream=stream)
            qm.bucket(ids, E, counts, offsets, perm, inv, scratch=bs, stream=stream)
            qm.stage_plan(counts, sm_res, first, window, slot_map_out=sm2, copy_list=cl,
                          counters=cnt, stream=stream)
            hip.record(copy_ev[li][0], stream.cuda_stream)
            qm.stage_copy(pool, backing, cl, cnt, first, window, stream=stream)
            hip.record(copy_ev[li][1], stream.cuda_stream)
            hip.record(ev[li][0], stream.cuda_stream)
            qm.expert_gate_up(pool, sm2, x, k, offsets, perm, h=h, stream=stream)
            hip.record(ev[li][1], stream.cuda_stream)
            qm.expert_down(pool, sm2, T, k, offsets, h, y=y, stream=stream)
            qm.combine(y, inv, w, out=outs[li], stream=stream)
        calls.append(call)
    return calls, copy_ev


def staged_overlap_calls(qm, torch, layers, staged, outs, cfg, resident, window, stream, hip,
                         ev):
    """Staged prefill with the bulk copy of each layer on a second stream, issued one layer
    ahead: while the compute stream runs layer l's expert FFN, the copy stream plans and
    copies layer l+1's window. The plan is made from a count of one per expert (every expert
    of a large prefill batch has pairs), so it needs no routing of its own and the copy can
    start before the layer's router runs. Each layer has its own pool, window and rewritten
    map, so the copy never writes slots a running GEMM reads. The compute stream waits on an
    event recorded after the layer's copy. Returns one callable per layer (the first also
    issues layer 0's copy) and the copy events."""
    T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
    dev = outs[0].device
    i32 = dict(dtype=torch.int32, device=dev)
    copy_stream = torch.cuda.Stream(device=dev)   # default priority, as the compute stream
    ids = torch.empty((T, k), **i32)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    perm, inv = torch.empty(T * k, **i32), torch.empty(T * k, **i32)
    rs = qm._scratch(qm.route_scratch_bytes(T, H, E), dev)
    bs = qm._scratch(qm.bucket_scratch_bytes(T, k, E), dev)
    every = torch.ones(E, **i32)
    n = len(layers)
    sm2 = [torch.empty(E, **i32) for _ in range(n)]
    cl = [torch.empty(E, **i32) for _ in range(n)]
    cnt = [torch.empty(2, **i32) for _ in range(n)]
    ready = [hip.create() for _ in range(n)]      # layer's window copied
    consumed = [hip.create() for _ in range(n)]   # layer's expert FFN done with its window
    h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    copy_ev = [(hip.create(), hip.create()) for _ in layers]
    first = len(resident)
    lib = hip.lib
    lib.hipStreamWaitEvent.argtypes = [hip.ct.c_void_p, hip.ct.c_void_p, hip.ct.c_uint]

    def wait(stream_, event):
        st = lib.hipStreamWaitEvent(hip.ct.c_void_p(stream_.cuda_stream), hip.ct.c_void_p(event), 0)
        if st != 0:
            raise RuntimeError(f"hipStreamWaitEvent failed ({st})")

    def issue_copy(li):
        pool = layers[li][0]
        backing, sm_res = staged[li]
        # the previous step's expert FFN of this layer must be done with the window (an event
        # not yet recorded, as on the first step, is no wait)
        wait(copy_stream, consumed[li])
        qm.stage_plan(every, sm_res, first, window, slot_map_out=sm2[li], copy_list=cl[li],
                      counters=cnt[li], stream=copy_stream)
        hip.record(copy_ev[li][0], copy_stream.cuda_stream)
        qm.stage_copy(pool, backing, cl[li], cnt[li], first, window, stream=copy_stream)
        hip.record(copy_ev[li][1], copy_stream.cuda_stream)
        hip.record(ready[li], copy_stream.cuda_stream)

    calls = []
    for li, (pool, x, wr, bias, _) in enumerate(layers):
        def call(pool=pool, x=x, wr=wr, bias=bias, li=li):
            if li == 0:
                issue_copy(0)
            if li + 1 < n:
                issue_copy(li + 1)
            qm.route(x, wr, bias, k, ids=ids, w=w, scratch=rs, stream=stream)
            qm.bucket(ids, E, counts, offsets, perm, inv, scratch=bs, stream=stream)
            wait(stream, ready[li])
            hip.record(ev[li][0], stream.cuda_stream)
            qm.expert_gate_up(pool, sm2[li], x, k, offsets, perm, h=h, stream=stream)
            hip.record(ev[li][1], stream.cuda_stream)
            qm.expert_down(pool, sm2[li], T, k, offsets, h, y=y, stream=stream)
            qm.combine(y, inv, w, out=outs[li], stream=stream)
            hip.record(consumed[li], stream.cuda_stream)
        calls.append(call)
    return calls, copy_ev


def library_sources_digest() -> str:
    """SHA-256 over the library's sources (kernels and the C ABI), in name order."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    files = [os.path.join(root, "include", "moe.h")]
    csrc = os.path.join(root, "quantized_routed_expert_gemv_amd", "csrc")
    files += sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel, from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE summary in profiles/ (each counter scaled by its reading on a copy of known
    size), or None when there is none for this workload or the kernels have changed since
    the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    digest = library_sources_digest()
    with open(path) as fh:
        for line in fh:
            if not line.startswith("traffic:"):
                continue
            kv = dict(item.split("=", 1) for item in line.split()[1:])
            if kv.get("workload") == workload and kv.get("sources") == digest:
                return int(kv["bytes"])
    return None


class HipEvents:
    """hipEvent_t handles through the HIP runtime that torch already loaded."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        # bind to the HIP runtime this process already uses (torch's and the library's):
        # loading another copy by name would give events that runtime does not know
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("no HIP runtime is loaded in this process")
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self) -> int:
        h = self.ct.c_void_p()
        st = self.lib.hipEventCreateWithFlags(self.ct.byref(h), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
        self.made.append(h.value)
        return h.value

    def capture(self, stream: int, fn):
        """Capture fn()'s launches on `stream` into an instantiated HIP graph."""
        ct, lib = self.ct, self.lib
        lib.hipStreamBeginCapture.argtypes = [ct.c_void_p, ct.c_int]
        lib.hipStreamEndCapture.argtypes = [ct.c_void_p, ct.POINTER(ct.c_void_p)]
        lib.hipGraphInstantiate.argtypes = [ct.POINTER(ct.c_void_p), ct.c_void_p, ct.c_void_p,
                                            ct.c_char_p, ct.c_size_t]
        GLOBAL = 0
        st = lib.hipStreamBeginCapture(ct.c_void_p(stream), GLOBAL)
        if st != 0:
            raise RuntimeError(f"hipStreamBeginCapture failed ({st})")
        try:
            fn()
        finally:
            g = ct.c_void_p()
            st = lib.hipStreamEndCapture(ct.c_void_p(stream), ct.byref(g))
        if st != 0:
            raise RuntimeError(f"hipStreamEndCapture failed ({st})")
        ge = ct.c_void_p()
        st = lib.hipGraphInstantiate(ct.byref(ge), g, None, None, 0)
        if st != 0:
            raise RuntimeError(f"hipGraphInstantiate failed ({st})")
        self.graphs = getattr(self, "graphs", []) + [(g, ge)]
        return ge.value

    def record(self, event: int, stream: int):
        self.lib.hipEventRecord.argtypes = [self.ct.c_void_p, self.ct.c_void_p]
        st = self.lib.hipEventRecord(self.ct.c_void_p(event), self.ct.c_void_p(stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def launch(self, graph_exec: int, stream: int):
        self.lib.hipGraphLaunch.argtypes = [self.ct.c_void_p, self.ct.c_void_p]
        st = self.lib.hipGraphLaunch(self.ct.c_void_p(graph_exec), self.ct.c_void_p(stream))
        if st != 0:
            raise RuntimeError(f"hipGraphLaunch failed ({st})")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self.ct.c_float()
        st = self.lib.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a), self.ct.c_void_p(b))
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value


def cpu_facts():
    """Cores this process may use, the CPU model and the BLAS numpy calls."""
    affinity = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return affinity, model, blas


def cpu_baseline(cfg, host_layers, budget_s):
    """The fp64 oracle on the host: 1 warm-up run, then the median of 3 timed runs, each a
    fixed number of whole-layer calls (decode) or 64-token slices (prefill) sized so the
    three take about `budget_s`. BLAS runs on every core of the process's affinity mask,
    up to the OMP_NUM_THREADS share the environment sets."""
    import numpy as np
    from oracle import moe as omoe
    affinity, model, blas = cpu_facts()
    cores = affinity
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        cores = max(1, min(cores, int(os.environ["OMP_NUM_THREADS"])))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limit = None
    T, k = cfg.T, cfg.k
    sample_T = min(T, 64)

    def one(i):
        L = host_layers[i % len(host_layers)]
        omoe.layer(L.planes, cfg.fmt, L.slot_map, L.wr, L.bias, L.x[:sample_T], k)

    t0 = time.perf_counter()
    one(0)                                       # warm-up, also sizes the runs
    per_call = time.perf_counter() - t0
    calls = max(1, int(budget_s / 3 / max(per_call, 1e-6)))
    runs = []
    for r in range(3):
        t0 = time.perf_counter()
        for i in range(calls):
            one(r * calls + i + 1)
        runs.append(time.perf_counter() - t0)
    if limit is not None:
        limit.restore_original_limits()
    med = sorted(runs)[1]
    sample = (f"median of 3 runs of {calls} layer call(s) x {sample_T} token(s) of {cfg.name} "
              "after 1 warm-up call; whole layer (route, bucket, dequantize the selected "
              "experts, FFN, combine) in fp64"
              + ("; prefill tokens/s extrapolated linearly from the slices" if T > sample_T else ""))
    return {"value": round(calls * sample_T / med, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "sample": sample, "seconds": round(sum(runs) + per_call, 2),
            "runs_s": [round(v, 3) for v in runs], "cpu_model": model, "blas": blas,
            "affinity_cores": affinity}


if __name__ == "__main__":
    main()
