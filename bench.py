#!/usr/bin/env python3
"""Benchmark of the decode-phase linear layer on one MI355X.

One step = one pass of the whole hot path over one batch: every linear of the
workload streamed once by the C-ABI library (main pass + deterministic
second pass), with inputs already resident in HBM.

Default workload: the Qwen2.5-72B decode linear stack at tensor-parallel
degree 1 and M = 1 token -- 80 layers x (QKV 10240x8192, O 8192x8192,
gate_up 59136x8192, down 8192x29568), bf16, distinct seeded weights
(140.4 GB), W ~ N(0, 0.02), x ~ N(0, 1).  Weights are made on the GPU by the
seeded input generator.

Printed: one JSON line with the contract fields, the dominant kernel's
roofline (HBM bytes / average main-kernel duration from HIP events recorded
around each launch on the library's stream) and the fp64 oracle timed on a
bounded sample on this host's cores.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "achieved HBM GB/s and % of 8 TB/s peak; µs per Qwen2.5-72B decode linear stack"

WORKLOADS = {
    "qwen2.5-72b-tp1-stack-bf16": "80 layers x (QKV 10240x8192, O 8192x8192, gate_up 59136x8192, "
                                  "down 8192x29568), bf16 W",
    "qwen2.5-72b-tp1-stack-fp8": "80 layers x TP=1 shapes, FP8-E4M3 W + 128x128 fp32 block scales",
    "qwen2.5-72b-tp8-layer-bf16": "one layer's TP=8 shard: QKV 1280x8192, O 8192x1024, "
                                  "gate_up 7392x8192, down 8192x3696, bf16 W",
    "qwen2.5-72b-tp8-qkv-gemv-bf16": "QKV shard GEMV 1280x8192, bf16 W",
    "qwen2.5-72b-lm-head-argmax-bf16": "vocabulary projection 152064x8192, bf16 W, then the greedy "
                                       "token of each row on the device",
    "qwen2.5-72b-tp1-mlp-swiglu-bf16": "one layer's gated MLP at TP=1: gate_up 59136x8192, silu(g)*u "
                                       "fused into down's input staging, down 8192x29568, bf16 W",
    "qwen2.5-72b-tp1-mlp-swiglu-fp8": "the same gated MLP with FP8-E4M3 W + 128x128 fp32 block scales",
    "moe-verify-experts-fp8": "MoE verify step: M tokens (default 6) routed to the top 2 of 8 "
                              "experts (two favoured), hidden 4096, expert width 1536: the "
                              "chosen experts' gate_up [3072x4096] then down [4096x1536] with "
                              "silu(g)*u fused, FP8-E4M3 W + 128x128 fp32 block scales",
    "moe-verify-experts-bf16": "the same MoE verify step with bf16 expert weights",
}


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="qwen2.5-72b-tp1-stack-bf16", choices=sorted(WORKLOADS))
    p.add_argument("--m", type=int, default=None,
                   help="tokens per step (1..16; default 1, the MoE verify step 6)")
    p.add_argument("--variant", default="auto", choices=["auto", "vector", "mfma"])
    p.add_argument("--waves", type=int, default=0, help="persistent waves (0 = automatic)")
    p.add_argument("--rotate-bytes", type=float, default=2.5e9,
                   help="small workloads cycle weight copies totalling at least this many bytes "
                        "so every step reads HBM, not the 256 MB last-level cache")
    p.add_argument("--batches", type=int, default=7,
                   help="event-bracketed batches inside the timed region (median / min / max)")
    p.add_argument("--read-reference-gib", type=int, default=8,
                   help="after timing, measure the HBM read ceiling on a buffer of this many "
                        "GiB: the streaming-read probe's patterns and PyTorch's int64 sum, "
                        "reported as context (0 = skip)")
    p.add_argument("--probe-only", action="store_true",
                   help="only measure the HBM read ceiling (the arithmetic-free streaming-read "
                        "probe and PyTorch's sum over the same buffer) and print it as JSON")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-rows", type=int, default=2048)
    p.add_argument("--calibration-copy-mib", type=int, default=0,
                   help="after timing, run one plain elementwise copy of this many MiB "
                        "(torch.neg into a second buffer): a kernel of known HBM traffic that "
                        "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return p.parse_args()


def make_workload(name):
    from gemv_skinny_gemm_amd import workloads as wl
    if name == "qwen2.5-72b-tp1-stack-bf16":
        return wl.tp1_stack(wl.BF16)
    if name == "qwen2.5-72b-tp1-stack-fp8":
        return wl.tp1_stack(wl.FP8_BS128)
    if name == "qwen2.5-72b-tp8-layer-bf16":
        return wl.tp8_layer(wl.BF16)
    if name == "qwen2.5-72b-tp8-qkv-gemv-bf16":
        return wl.qkv_tp8_gemv()
    if name == "qwen2.5-72b-lm-head-argmax-bf16":
        return wl.lm_head(wl.BF16)
    if name == "qwen2.5-72b-tp1-mlp-swiglu-bf16":
        return wl.mlp(1, wl.BF16)
    if name == "qwen2.5-72b-tp1-mlp-swiglu-fp8":
        return wl.mlp(1, wl.FP8_BS128)
    if name == "moe-verify-experts-fp8":
        return wl.moe_experts(wl.FP8_BS128)
    if name == "moe-verify-experts-bf16":
        return wl.moe_experts(wl.BF16)
    raise ValueError(name)


def moe_routes(M):
    """The verify step's seeded router choices (int32 [M][top k])."""
    from gemv_skinny_gemm_amd import synth
    from gemv_skinny_gemm_amd import workloads as wl
    return synth.route_topk(0, synth.stream_id("moe-verify", M), M, wl.MOE_EXPERTS, wl.MOE_TOPK)


def moe_bytes(specs, ids):
    """(gate_up call, down call) algorithmic bytes: chosen experts' W once."""
    from gemv_skinny_gemm_amd import workloads as wl
    gu, dn = specs
    E = wl.MOE_EXPERTS
    a = wl.moe_algorithmic_bytes(gu, ids, E, ids.shape[0], gu.K)
    b = wl.moe_algorithmic_bytes(dn, ids, E, ids.size, 2 * dn.K)
    return a, b


def step_work(specs, M, ids=None):
    """(flops, weight bytes) of one step: 2 M N K per linear and every weight
    and scale byte once; for a mixture-of-experts step (ids = the routes'
    experts), 2 flops per (route, output, k) and only the chosen experts'
    weights."""
    from gemv_skinny_gemm_amd import workloads as wl
    if ids is None:
        return wl.flops(specs, M), sum(s.weight_bytes() + s.scale_bytes() for s in specs)
    E = wl.MOE_EXPERTS
    flat = [int(e) for e in ids.ravel()]
    chosen = len({e for e in flat if 0 <= e < E})
    routes = sum(1 for e in flat if 0 <= e < E)
    flops = sum(2 * routes * (s.N // E) * s.K for s in specs)
    return flops, sum(chosen * ((s.weight_bytes() + s.scale_bytes()) // E) for s in specs)


def moe_cpu_baseline(specs, ids, seed=0):
    """The fp64 oracle over the whole MoE step (it is small): gate_up, then
    down on the oracle's own bf16 gate_up outputs.  Returns seconds, bytes,
    threads, (g_ref, g_a, the down experts' weights and scales) and a
    description."""
    import numpy as np

    import oracle
    from gemv_skinny_gemm_amd import synth
    from gemv_skinny_gemm_amd import workloads as wl

    E, T = wl.MOE_EXPERTS, ids.shape[0]
    gu, dn = specs
    x = synth.tensor_bf16(seed, gu.x_stream, T, gu.K, wl.X_SIGMA)
    ws = []
    for s in specs:
        if s.dtype == wl.BF16:
            ws.append((synth.tensor_bf16(seed, s.w_stream, s.N, s.K, wl.W_SIGMA)
                       .reshape(E, s.N // E, s.K), None))
        else:
            q, sc, _ = synth.fp8_weight_bs128(seed, s.w_stream, s.N, s.K, wl.W_SIGMA)
            ws.append((q.reshape(E, s.N // E, s.K), sc.reshape(E, -1, sc.shape[1])))
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        g_ref, g_a = oracle.moe_linear(x, ids, ws[0][0], scales=ws[0][1])
        h = oracle.bf16_encode(g_ref)
        oracle.moe_linear(h, ids, ws[1][0], scales=ws[1][1], x_per_route=True, swiglu=True)
        times.append(time.perf_counter() - t0)
    secs = float(np.median(times))
    desc = (f"the whole step ({T} tokens, {ids.size} routes, gate_up then down), compute only, "
            "median of 3 runs")
    return secs, sum(moe_bytes(specs, ids)), oracle.host_threads(), (g_ref, g_a, ws[1]), desc


def measured_traffic(workload, M):
    """HBM bytes per main launch from the committed rocprofv3 counter summary,
    or None when there is none for this workload or the kernels changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    try:
        t = json.load(open(path))
        src = os.path.join(ROOT, t["kernel_source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != t["kernel_source_sha256"]:
            return None
        e = t["entries"].get(f"{workload}/M{M}")
        return int(e["traffic_bytes_per_launch"]) if e else None
    except (OSError, ValueError, KeyError):
        return None


def calibrate_spin(stream):
    """GPU spin-kernel cycles per millisecond (torch.cuda._sleep)."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    n = 1_000_000
    torch.cuda._sleep(n)
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(n)
    b.record(stream)
    torch.cuda.synchronize()
    return n / max(a.elapsed_time(b), 1e-3)


def cpu_baseline(specs, M, rows, seed=0, repeats=5):
    """The fp64 oracle on a bounded sample: the first `rows` rows of each linear
    of the first layer, from the same seeded streams.  Returns the result
    dict, the sampled reference outputs and the sample description."""
    import numpy as np

    import oracle
    from gemv_skinny_gemm_amd import synth
    from gemv_skinny_gemm_amd import workloads as wl

    layer = specs[:4] if len(specs) >= 4 else specs
    total_s, total_b, refs, threads = 0.0, 0, [], 0
    for s in layer:
        r = min(rows, s.N)
        x = synth.tensor_bf16(seed, s.x_stream, M, s.K, wl.X_SIGMA)
        times = []
        if s.dtype == wl.BF16:
            w = synth.tensor_bf16(seed, s.w_stream, r, s.K, wl.W_SIGMA)
            for _ in range(repeats):
                t0 = time.perf_counter()
                y, a, threads = oracle.linear_bf16(x, w)
                times.append(time.perf_counter() - t0)
            total_b += r * s.K * 2
        else:
            bands = (r + 127) // 128
            q, sc, _ = synth.fp8_weight_bs128(seed, s.w_stream, s.N, s.K, wl.W_SIGMA, 0, bands)
            q, r = q[:r], min(r, q.shape[0])
            scr = sc[:(r + 127) // 128]
            for _ in range(repeats):
                t0 = time.perf_counter()
                y, a, threads = oracle.linear_fp8_bs128(x, q, scr)
                times.append(time.perf_counter() - t0)
            total_b += r * s.K + scr.size * 4
        total_s += float(np.median(times))
        total_b += 2 * M * s.K + 2 * M * r
        refs.append((s, r, y, a))
    desc = (f"first {rows} rows of each of the {len(layer)} linears of layer 0 "
            f"({total_b / 1e6:.1f} MB of algorithmic bytes), compute only, median of "
            f"{repeats} runs")
    return total_s, total_b, threads, refs, desc


# The streaming-read probe's configurations (gemv_skinny_gemm_amd/probe):
# (label, order, row bytes, KB per batch, waves per CU, nontemporal loads).
# Measured on MI355X over orders, row sizes, batch depths and grid sizes,
# reads stream fastest with about 32 KB in flight per CU in a compact window
# of addresses, and nontemporal loads (the hint the library's weight loads
# carry) stream ~10% faster than plain ones; the plain deep row-streaming
# pattern (16 waves per CU, 8 KB batches) is kept for contrast.
PROBE_CONFIGS = [
    ("32 KB rows to 4-wave workgroups, waves interleaving 2 KB batches, 8 waves/CU, "
     "nontemporal loads", 1, 32 << 10, 2, 8, True),
    ("8 KB rows to waves, 2 KB batches, 8 waves/CU, nontemporal loads", 0, 8 << 10, 2, 8, True),
    ("32 KB rows to 4-wave workgroups, waves interleaving 2 KB batches, 8 waves/CU",
     1, 32 << 10, 2, 8, False),
    ("8 KB rows to waves, 2 KB batches, 8 waves/CU", 0, 8 << 10, 2, 8, False),
    ("16 KB rows to waves, 8 KB batches, 16 waves/CU", 0, 16 << 10, 8, 16, False),
]


def read_ceiling(gib: int, stream) -> dict:
    """The HBM read ceiling on this GPU: the probe's configurations and
    PyTorch's reduction kernel, each streaming the same buffer of `gib` GiB
    (10 timed passes after 2 untimed ones)."""
    import torch
    from gemv_skinny_gemm_amd import probe
    n = gib << 30
    t = torch.ones(n // 8, dtype=torch.int64, device="cuda")
    out = {"bytes": n, "probe": []}
    for label, order, row, u, wpc, nt in PROBE_CONFIGS:
        gbps = probe.measure(t, row, order, u, wpc, reps=10, nontemporal=nt)
        out["probe"].append({"pattern": label, "gbps": round(gbps, 1)})
    out["probe_best_gbps"] = max(p["gbps"] for p in out["probe"])
    for _ in range(3):
        t.sum()
    torch.cuda.synchronize()
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(10):
        t.sum()
    r1.record(stream)
    torch.cuda.synchronize()
    out["torch_sum_gbps"] = round(n / (r0.elapsed_time(r1) / 10 * 1e-3) / 1e9, 1)
    out["what"] = ("arithmetic-free streaming reads (gemv_skinny_gemm_amd/probe) and PyTorch's "
                   "int64 sum over the same buffer: the HBM read ceiling this library is held "
                   "against, not this library")
    del t
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the decode linear "
                                   "stack is measured at one GPU's share; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    moe = args.workload.startswith("moe-")
    if args.m is None:
        args.m = 6 if moe else 1
    if not 1 <= args.m <= 16:
        sys.exit("--m must be in 1..16")

    import numpy as np
    import torch

    import gemv_skinny_gemm_amd as sg
    from gemv_skinny_gemm_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.probe_only:
        gib = args.read_reference_gib or 8
        print(json.dumps({"read_ceiling": read_ceiling(gib, torch.cuda.current_stream()),
                          "gpu": torch.cuda.get_device_name(0)}), flush=True)
        return
    sg.lib()
    M = args.m
    specs = make_workload(args.workload)
    head = args.workload.startswith("qwen2.5-72b-lm-head")
    mlp = "-mlp-" in args.workload
    # The greedy token adds M int32 outputs to the step's bytes; a gated MLP
    # counts its [M][2I] intermediate written and read.
    if mlp:
        step_bytes = wl.mlp_algorithmic_bytes(specs, M)
    elif moe:
        ids_host = moe_routes(M)
        moe_gu_bytes, moe_dn_bytes = moe_bytes(specs, ids_host)
        step_bytes = moe_gu_bytes + moe_dn_bytes
    else:
        step_bytes = wl.algorithmic_bytes(specs, M) + (4 * M if head else 0)
    step_flops, step_weight_bytes = step_work(specs, M, ids_host if moe else None)
    copies = 1 if step_bytes >= args.rotate_bytes else int(np.ceil(args.rotate_bytes / step_bytes))
    log(f"workload {args.workload}: {len(specs)} linears, M={M}, {step_bytes / 1e9:.3f} GB/step, "
        f"{copies} rotating cop{'y' if copies == 1 else 'ies'}")
    t0 = time.perf_counter()
    from gemv_skinny_gemm_amd.synth import gpu as sgpu
    sets, tensors = sgpu.materialise(specs, M, copies)
    log(f"inputs made on the GPU in {time.perf_counter() - t0:.1f} s")

    variant = {"auto": sg.VARIANT_AUTO, "vector": sg.VARIANT_VECTOR, "mfma": sg.VARIANT_MFMA}[args.variant]
    if mlp:
        mlps = [sg.make_mlp(t[0][0], t[0][1], t[1][1], t[1][3], t[0][2], t[1][2]) for t in tensors]
        ws = torch.empty(sg.mlp_workspace_bytes(mlps[0], M), dtype=torch.uint8, device="cuda")
    elif moe:
        E = wl.MOE_EXPERTS
        ids = torch.from_numpy(ids_host).cuda()

        def experts(t):
            w, sc = t[1], t[2]
            return sg.make_experts(w.view(E, w.shape[0] // E, w.shape[1]),
                                   None if sc is None else sc.view(E, -1, sc.shape[1]))
        moe_ex = [(experts(t[0]), experts(t[1])) for t in tensors]
        routes = ids_host.size
        moe_y = torch.empty((routes, specs[1].N // E), dtype=torch.bfloat16, device="cuda")
        # Zeroed: the one-token launch keeps its counters at the workspace's
        # start; the gate_up outputs follow them.
        ws = torch.zeros(sg.moe_mlp_workspace_bytes(moe_ex[0][0], moe_ex[0][1], M, wl.MOE_TOPK),
                         dtype=torch.uint8, device="cuda")
        n_gu = specs[0].N // E
        c0 = sg.MOE_MLP_COUNTER_BYTES
        one_launch = sg.moe_mlp_plan_query(moe_ex[0][0], moe_ex[0][1], M, wl.MOE_TOPK).kernel == 7

        def moe_gate_up():
            """The gate_up outputs the last call left in the workspace (one
            launch: 64-bit words, a call number above two bf16 outputs)."""
            if one_launch:
                w = ws[c0:c0 + routes * n_gu * 4].view(torch.int32).view(routes, n_gu // 2, 2)
                return w[:, :, 0].contiguous().view(torch.bfloat16).view(routes, n_gu)
            return ws[c0:c0 + routes * n_gu * 2].view(torch.bfloat16).view(routes, n_gu)
    else:
        ws = torch.empty(sg.stack_workspace_bytes(sets[0], M), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # The dominant kernel: the stack's main launches, or an MLP's gate_up
    # launch (two thirds of its bytes), timed through the same entry point.
    timed_sets = [st[:1] for st in sets] if mlp else sets
    timed_bytes = wl.algorithmic_bytes(specs[:1], M) if mlp else step_bytes
    if moe:
        # The MoE step's dominant kernel: its one launch (one token), else its
        # gate_up launch (two thirds of the bytes).
        plan = sg.moe_mlp_plan_query(moe_ex[0][0], moe_ex[0][1], M, wl.MOE_TOPK)
        timed_bytes = step_bytes if sg.KERNEL_NAMES.get(plan.kernel) == "skinny_moe_mlp1" \
            else moe_gu_bytes
        n_launch = 1
    else:
        plan = sg.plan_query(timed_sets[0], M)
        n_launch = sg.launch_count(timed_sets[0])

    tokens = [torch.zeros(M, dtype=torch.int32, device="cuda") for _ in range(copies)]

    def step(i):
        if moe:
            ex_gu, ex_dn = moe_ex[i % copies]
            sg.moe_mlp_swiglu(ex_gu, ex_dn, tensors[i % copies][0][0], ids, moe_y, ws)
            return
        if head or mlp:
            if variant != sg.VARIANT_AUTO or args.waves:
                sys.exit("the lm-head and MLP workloads run the automatic plan")
        if head:
            sg.lm_head_argmax(sets[i % copies][0], M, tokens[i % copies], ws)
        elif mlp:
            sg.mlp_swiglu(mlps[i % copies], M, ws)
        else:
            sg.linear_run(sets[i % copies], M, ws, variant=variant, waves=args.waves)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # A GPU spin kernel ahead of each timed region keeps the stream busy while
    # the host enqueues, so the timed launches run back to back on the GPU
    # and host launch overhead stays out of the figures.
    spin_cycles = calibrate_spin(stream)

    # The host enqueues each timed region while a spin kernel holds the GPU;
    # a garbage-collector pass in the middle (tens of ms in a process holding
    # torch) could outlast that lead and show up as GPU idle time, so the
    # collector stays off until the timed regions are done.
    gc.collect()
    gc.disable()

    # The spin that leads a timed region is sized from the host's enqueue
    # time and the GPU's time per step, both measured here on untimed steps:
    # long enough for the host to stay ahead of the GPU, and no longer, since
    # a GPU left near idle for many milliseconds runs the next steps at a
    # transiently lower rate (measured on MI355X: the TP=8 layer at M = 4 on
    # the flat row kernel took 44 us per step after a 1 ms lead but rose to
    # 49 us within 5 ms of steps after a 15 ms one).
    n_cal = max(5, min(50, args.steps))
    t0 = time.perf_counter()
    for i in range(n_cal):
        step(args.warmup + i)
    host_ms = (time.perf_counter() - t0) * 1e3 / n_cal
    torch.cuda.synchronize()
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(spin_cycles * (1.0 + 2.0 * n_cal * host_ms)))
    ca.record(stream)
    for i in range(n_cal):
        step(args.warmup + i)
    cb.record(stream)
    torch.cuda.synchronize()
    gpu_ms = ca.elapsed_time(cb) / n_cal

    def prefill(n, host_factor=1.0):
        """Spin ahead of n steps whose enqueue costs host_factor x host_ms each."""
        lag = n * max(0.0, 1.5 * host_factor * host_ms - gpu_ms)
        torch.cuda._sleep(int(spin_cycles * (1.0 + lag)))

    # Timed region: K whole steps between two events on the library's stream,
    # with events between batches of steps (up to 7) for the spread.
    nb = max(1, min(args.batches, args.steps))
    bounds = [b * args.steps // nb for b in range(nb + 1)]
    bev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    prefill(args.steps)
    bev[0].record(stream)
    for b in range(nb):
        for i in range(bounds[b], bounds[b + 1]):
            step(args.warmup + i)
        bev[b + 1].record(stream)
    torch.cuda.synchronize()
    ms_per_step = bev[0].elapsed_time(bev[nb]) / args.steps
    batch_us = [bev[b].elapsed_time(bev[b + 1]) / (bounds[b + 1] - bounds[b]) * 1e3
                for b in range(nb)]
    log(f"{ms_per_step * 1e3:.1f} us/step")

    # Hot-cache figure (labelled, never the value): the same steps on weight
    # copy 0 only, so a workload smaller than the 256 MB last-level cache can
    # be served from it.
    hot_us = None
    if copies > 1:
        h0 = torch.cuda.Event(enable_timing=True)
        h1 = torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            step(0)
        torch.cuda.synchronize()
        prefill(args.steps)
        h0.record(stream)
        for _ in range(args.steps):
            step(0)
        h1.record(stream)
        torch.cuda.synchronize()
        hot_us = h0.elapsed_time(h1) / args.steps * 1e3

    # Dominant kernel: events recorded by the library around every main launch.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_launch * args.steps)]
    for e in evs:
        e.record(stream)                     # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    prefill(args.steps, host_factor=2.0)
    for i in range(args.steps):
        handles = [e.cuda_event for e in evs[2 * n_launch * i: 2 * n_launch * (i + 1)]]
        if moe:
            c = (args.warmup + i) % copies
            sg.moe_mlp_swiglu_timed(moe_ex[c][0], moe_ex[c][1], tensors[c][0][0], ids, moe_y, ws,
                                    handles)
            continue
        sg.linear_run_timed(timed_sets[(args.warmup + i) % copies], M, ws, handles,
                            variant=variant, waves=args.waves)
    torch.cuda.synchronize()
    gc.enable()
    main_ms = [evs[2 * k].elapsed_time(evs[2 * k + 1]) for k in range(n_launch * args.steps)]
    main_avg_ms = float(np.mean(main_ms))
    bytes_per_launch = timed_bytes / n_launch
    achieved = bytes_per_launch / (main_avg_ms * 1e-3) / 1e9
    main_total_ms = float(np.sum(main_ms)) / args.steps

    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if specs[0].dtype == wl.BF16 else "fp8e4m3 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded Philox4x32-10; W ~ N(0,0.02), x ~ N(0,1), bf16-rounded)",
        "config": {
            "workload": args.workload,
            "description": WORKLOADS[args.workload],
            "M": M,
            "linears": len(specs),
            "algorithmic_bytes_per_step": step_bytes,
            "flops_per_step": step_flops,
            "us_per_step": round(ms_per_step * 1e3, 2),
            "us_per_step_batches": {"batches": nb, "us": [round(b, 2) for b in batch_us],
                                    "median": round(float(np.median(batch_us)), 2),
                                    "min": round(min(batch_us), 2), "max": round(max(batch_us), 2)},
            "hot_cache_us_per_step": None if hot_us is None else round(hot_us, 2),
            "lead_in": {"host_us_per_step": round(host_ms * 1e3, 2),
                        "gpu_us_per_step": round(gpu_ms * 1e3, 2)},
            "pct_of_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 2),
            # Weight-only MBU: weight (and scale) bytes per second over the peak,
            # the decode figure of "Developing a custom Qwen2.5 72B inference
            # engine from scratch", section 6.1.
            "weight_only_mbu_pct": round(
                100 * step_weight_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
            "tflops": round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
            "weight_copies_rotated": copies,
            "variant": {0: "auto", 1: "vector", 2: "mfma"}[variant],
            "auto_plan": {"variant": {1: "vector", 2: "mfma"}.get(plan.variant, plan.variant),
                          "waves": plan.waves, "kernel": sg.KERNEL_NAMES.get(plan.kernel)},
            "main_launches_per_step": n_launch,
            "gpu": torch.cuda.get_device_name(0),
        },
        "roofline": {
            "kernel": (sg.KERNEL_NAMES.get(plan.kernel, "skinny_main") if variant == sg.VARIANT_AUTO
                       else {1: "skinny_rows", 2: "skinny_tiles"}.get(variant, "skinny_main")),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(args.workload, M),
            "avg_launch_us": round(main_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
            "main_us_per_step": round(main_total_ms * 1e3, 2),
        },
    }

    if args.read_reference_gib:
        rc = read_ceiling(args.read_reference_gib, stream)
        result["config"]["read_ceiling"] = rc
        result["config"]["pct_of_read_ceiling"] = round(100 * gbps / rc["probe_best_gbps"], 1)

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 19                 # bf16 elements
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        result["config"]["calibration_copy_bytes"] = 2 * n
        del src, dst

    if moe:
        result["config"].update({
            "experts": wl.MOE_EXPERTS, "top_k": wl.MOE_TOPK, "routes": int(ids_host.size),
            "experts_chosen": len(set(ids_host.ravel().tolist())),
            "gate_up_bytes": moe_gu_bytes, "down_bytes": moe_dn_bytes})
        if one_launch:
            # A wait that gave up leaves wrong outputs: the run is then invalid.
            gave_up = sg.moe_mlp_gave_up(ws)
            result["config"]["one_launch_wait_gave_up"] = gave_up
            if gave_up:
                log("a wait of the one-launch MoE MLP gave up: outputs of this run are invalid")

    if not args.no_cpu_baseline and moe:
        import oracle
        secs, sbytes, threads, (g_ref, g_a, (wd, sd)), desc = moe_cpu_baseline(specs, ids_host)
        step(0)
        torch.cuda.synchronize()
        moe_gu = moe_gate_up()
        ok, worst, _ = oracle.check(moe_gu.float().cpu().double().numpy(), g_ref, g_a)
        if not ok:
            log(f"GPU gate_up output outside the bound (worst {worst:.3g})")
        # down against the oracle on the GPU's own gate_up outputs.
        h = moe_gu.cpu().view(torch.int16).numpy().view(np.uint16)
        d_ref, d_a = oracle.moe_linear(h, ids_host, wd, scales=sd, x_per_route=True, swiglu=True)
        ok_d, worst_d, _ = oracle.check(moe_y.float().cpu().double().numpy(), d_ref, d_a)
        if not ok_d:
            log(f"GPU down output outside the bound (worst {worst_d:.3g})")
        worst = max(worst, worst_d)
        result["cpu_baseline"] = {
            "value": round(sbytes / secs / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": desc, "us_per_step": round(secs * 1e6, 1),
            "cpu": cpu_model()}
        result["config"]["sampled_outputs_worst_err_over_bound"] = round(worst, 4)
    elif not args.no_cpu_baseline:
        import oracle
        secs, sbytes, threads, refs, desc = cpu_baseline(specs, M, args.cpu_sample_rows)
        cpu_gbps = sbytes / secs / 1e9
        # The oracle's sample also spot-checks the GPU outputs of step copy 0.
        step(0)
        torch.cuda.synchronize()
        worst = 0.0
        # (An MLP's linears run chained, so their outputs are not the sample's.)
        for (s, r, y_ref, a), t in zip([] if mlp else refs, tensors[0][:len(refs)]):
            yv = t[3][:, :r].float().cpu().double().numpy()
            ok, wr, _ = oracle.check(yv, y_ref, a)
            worst = max(worst, wr)
            if not ok:
                log(f"GPU output of {s.name} outside the bound (worst {wr:.3g})")
        result["cpu_baseline"] = {
            "value": round(cpu_gbps, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": desc,
            "us_per_step_extrapolated": round(step_bytes / (cpu_gbps * 1e9) * 1e6, 1),
            "cpu": cpu_model(),
        }
        result["config"]["sampled_outputs_worst_err_over_bound"] = round(worst, 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
