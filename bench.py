#!/usr/bin/env python3
"""Benchmark of the W4A16 MoE hot path on one MI355X.

One step = one fused expert-MLP call on synthetic inputs already resident in
HBM: routing preparation, gate_up grouped GEMM with SiLU*mul in its epilogue,
down grouped GEMM and the weighted top-k combine.  The default workload is the
largest one-GPU configuration: the DeepSeek-V3-shaped layer (256 experts,
top-8 of a softmax router, hidden 7168, intermediate 2048) at 4096 tokens,
128 routed rows per expert, whose gate_up GEMM is bound by the matrix cores.
Decode workloads (e.g. the Qwen3-30B-A3B-shaped layer at 64 tokens) are
selected with --workload.

Every step reads a different copy of the packed weights from a rotation pool
of at least 1 GiB, larger than the 256 MiB Infinity Cache plus the L2s, so the
weights come from HBM as they would in serving.

Prints one JSON line: the metric (effective weight GB/s of the step, i.e.
packed weight bytes of the experts that received a route divided by the step
time, from HIP-graph replays of the fused call), the roofline of the dominant
kernel (the gate_up GEMM, timed with HIP events recorded between the stages of
as many eager calls of the same step, queued behind a GPU sleep so that the
events bracket GPU work only), and the CPU oracle timed on the host on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "us/call + effective weight GB/s (% HBM peak), W4A16 MoE grouped GEMM"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense BF16 matrix peak of the MI355X
ROTATION_BYTES = 1 << 30
COPY_CAL_BYTES = 256 << 20


def workload_spec(name: str) -> dict:
    """Shapes and routing of a named workload."""
    import synth

    def qwen3(T):
        return dict(E=128, k=8, H=2048, I=768, T=T, cfg=2, routes=lambda: synth.qwen3_routes(T),
                    desc="Qwen3-30B-A3B-shaped MoE layer: 128 experts, top-8 uniform, hidden 2048, "
                         "intermediate 768, %d tokens" % T)

    def kimi(T):
        return dict(E=48, k=8, H=7168, I=2048, T=T, cfg=3, global_experts=384, routes=lambda: synth.kimi_decode_routes(T),
                    desc="Kimi-K2-shaped one-GPU expert share: 48 local of 384 experts, top-8 uniform "
                         "(about 1/8 of routes local), hidden 7168, intermediate 2048, %d tokens" % T)

    def deepseek(T):
        # the router's ids and weights come from one draw
        r = {}

        def draw():
            if not r:
                r["ids"], r["tw"] = synth.deepseek_router(T)
            return r

        return dict(E=256, k=8, H=7168, I=2048, T=T, cfg=5, device_weights=True, routes=lambda: draw()["ids"],
                    router_weights=lambda: draw()["tw"],
                    desc="DeepSeek-V3-shaped fused expert MLP on one GPU: 256 experts, top-8 of a softmax "
                         "router over seeded BF16 logits, hidden 7168, intermediate 2048, %d tokens" % T)

    def kimi_prefill(T):
        return dict(E=48, k=8, H=7168, I=2048, T=T, cfg=4, global_experts=384, device_weights=True,
                    routes=lambda: synth.kimi_prefill_routes(T),
                    desc="Kimi-K2-shaped one-GPU prefill share: 48 local of 384 experts, top-8 with Zipf(1.1) "
                         "expert popularity (about 1/8 of routes local, some local experts empty), hidden 7168, "
                         "intermediate 2048, %d tokens" % T)

    table = {}
    for T in (1, 8, 64, 512):
        table["qwen3-moe-t%d" % T] = qwen3(T)
    for T in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        table["kimi-moe-t%d" % T] = kimi(T)
    for T in (1, 32, 512, 4096):
        table["deepseek-moe-t%d" % T] = deepseek(T)
    table["kimi-prefill-t8192"] = kimi_prefill(8192)
    # the same layers with MXFP4 weights (E2M1 codes, E8M0 scales per 32 k)
    for key in list(table):
        mx = dict(table[key])
        mx["fmt"] = "mxfp4"
        mx["desc"] = mx["desc"] + "; MXFP4 weights"
        table[key + "-mxfp4"] = mx
    if name not in table:
        raise SystemExit("unknown workload %s; choose from %s" % (name, ", ".join(sorted(table))))
    spec = table[name]
    spec["name"] = name
    return spec


def packed_weight_bytes(N: int, K: int, fmt: str = "int4") -> int:
    # 16-row x 256-k superblocks: 2304 bytes with BF16 scales (4.5 bits per weight), 2176 with E8M0 scales
    # (4.25 bits per weight), when N % 16 == 0 and K % 256 == 0
    return ((N + 15) // 16) * ((K + 255) // 256) * (2176 if fmt == "mxfp4" else 2304)


def gate_up_algorithmic_bytes(spec, block_m: int = 16) -> int:
    """Bytes the gate_up GEMM (SiLU*mul epilogue) must move at least: the packed weights of every expert that
    received a route, x once, h written once, and the routing tensors read once."""
    from weight_only_int4_amd import lib as L

    E, k, H, I, T = spec["E"], spec["k"], spec["H"], spec["I"], spec["T"]
    flat = spec["routes"]().reshape(-1)
    valid = (flat >= 0) & (flat < E)
    active = len(np.unique(flat[valid]))
    maxP, maxB = L.route_bounds(T, k, E, block_m)
    return active * packed_weight_bytes(2 * I, H, spec.get("fmt", "int4")) + T * H * 2 + int(valid.sum()) * I * 2 + (maxP + maxB) * 4


def roofline_bound(spec, block_m: int = 16):
    """The roofline that bounds the gate_up launch: "hbm" or "mfma", whichever of its minimum HBM time
    (algorithmic bytes at the HBM peak) and its minimum matrix time (2 * valid routes * 2I * H flops at the
    dense BF16 peak) is longer, with both figures.  The kernel that runs does not decide it: a prefill plan at
    16 rows per expert streams its weights at a few flops per byte and is HBM-bound."""
    E, H, I = spec["E"], spec["H"], spec["I"]
    flat = spec["routes"]().reshape(-1)
    Rv = int(((flat >= 0) & (flat < E)).sum())
    alg_bytes = gate_up_algorithmic_bytes(spec, block_m)
    alg_flops = 2.0 * Rv * (2 * I) * H
    mfma = alg_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9)
    return ("mfma" if mfma else "hbm"), alg_bytes, alg_flops


# the sources the gate_up kernel of each family is built from
KERNEL_SOURCES = {
    "decode": ("weight_only_int4_amd/csrc/gemm_decode_reg.hip", "weight_only_int4_amd/csrc/gemm_decode.hip",
               "weight_only_int4_amd/csrc/decode_common.h", "weight_only_int4_amd/csrc/frag.h",
               "weight_only_int4_amd/csrc/w4a16_internal.h"),
    "prefill": ("weight_only_int4_amd/csrc/gemm_prefill.hip", "weight_only_int4_amd/csrc/frag.h",
                "weight_only_int4_amd/csrc/w4a16_internal.h"),
}


def kernel_sources_sha256(family: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str, family: str):
    """HBM bytes per launch of the gate_up kernel from the committed counter summary of this workload, or None
    when there is none or the kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "gate_up_silu_%s_hbm_traffic.md" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("|", "#", "`")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("workload") != workload or fields.get("kernel_sources_sha256") != kernel_sources_sha256(family):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_inputs(spec, dev=None):
    """x, ids, topk weights and the two weight sets: numpy arrays (codes uint8, scales BF16 bits or E8M0
    bytes), or, for weight sets of gigabytes, torch tensors drawn on the GPU (codes uint8, scales bfloat16 or
    uint8)."""
    import synth

    E, k, H, I, T = spec["E"], spec["k"], spec["H"], spec["I"], spec["T"]
    mx = spec.get("fmt") == "mxfp4"
    rng = synth.rng_for(spec["cfg"], 7)
    x = synth.activations(rng, T, H)
    if spec.get("device_weights"):
        base = 1000 * spec["cfg"]
        sdev = synth.mxfp4_scales_device if mx else synth.scales_device
        c13, s13 = synth.codes_device(base + 1, E, 2 * I, H, dev), sdev(base + 2, E, 2 * I, H, dev)
        c2, s2 = synth.codes_device(base + 3, E, H, I, dev), sdev(base + 4, E, H, I, dev)
    else:
        c13, s13 = synth.expert_weights(spec["cfg"], E, 2 * I, H, salt=1)
        c2, s2 = synth.expert_weights(spec["cfg"], E, H, I, salt=2)
        if mx:
            s13 = synth.mxfp4_scales(synth.rng_for(spec["cfg"], 201), E, 2 * I, H)
            s2 = synth.mxfp4_scales(synth.rng_for(spec["cfg"], 202), E, H, I)
    ids = spec["routes"]()
    if "router_weights" in spec:
        tw = spec["router_weights"]()
    else:
        tw = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
        tw /= tw.sum(axis=1, keepdims=True)
    return x, ids, tw, c13, s13, c2, s2


def host_expert_subset(ids, E, weights, max_experts):
    """For an oracle run on weights held on the GPU: the longest prefix of tokens whose local experts number
    at most ``max_experts``, those experts' weights copied to the host, and the ids renumbered to them."""
    import torch

    Ts, seen = 0, set()
    for t in range(ids.shape[0]):
        row = {int(e) for e in ids[t] if 0 <= e < E}
        if len(seen | row) > max_experts and Ts > 0:
            break
        seen |= row
        Ts += 1
    used = np.array(sorted(seen), np.int64)
    remap = np.full(E, -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    sub_ids = np.where((ids[:Ts] >= 0) & (ids[:Ts] < E), remap[np.clip(ids[:Ts], 0, E - 1)], -1).astype(np.int32)
    idx = torch.from_numpy(used).to(weights[0].device)
    host = []
    for w in weights:
        t = w.index_select(0, idx).cpu()
        host.append(t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy())
    return Ts, sub_ids, host


# Host threads one GPU's job may keep busy on the GPU machine: its CPU share is 16 threads whatever the
# machine's count of CPUs shows, so the oracle's pool is capped there.
CPU_SHARE_THREADS = 16


def available_cpus() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def oracle_threads() -> int:
    """Threads of the oracle's pool: every CPU this process may run on, up to the GPU job's CPU share."""
    return max(1, min(CPU_SHARE_THREADS, available_cpus()))


def cpu_baseline(spec, inputs, weight_bytes_step, budget_s=10.0):
    """The oracle (test infrastructure, never the product) timed on the host's cores on this workload."""
    import oracle

    x, ids, tw, c13, s13, c2, s2 = inputs
    o = oracle.Oracle(oracle.build())
    threads = oracle_threads()
    T = spec["T"]
    if spec.get("device_weights"):
        # weights live on the GPU: the oracle gets the tokens whose experts fit a host copy of 64 experts
        Tmax, ids, (c13, s13, c2, s2) = host_expert_subset(ids, spec["E"], (c13, s13, c2, s2), 64)
        x, tw = x[:Tmax], tw[:Tmax]
    # whole steps when one fits the budget, else the first Ts tokens, extrapolated linearly in tokens
    t0 = time.perf_counter()
    fmt = spec.get("fmt", "int4")
    o.fused_moe(x[:1], ids[:1], tw[:1], c13, s13, c2, s2, nthreads=threads, fmt=fmt)
    one_tok = max(time.perf_counter() - t0, 1e-3)
    Ts = T if one_tok * T <= 3 * budget_s else max(1, int(budget_s / one_tok))
    Ts = min(Ts, ids.shape[0])
    times = []
    start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        o.fused_moe(x[:Ts], ids[:Ts], tw[:Ts], c13, s13, c2, s2, nthreads=threads, fmt=fmt)
        times.append(time.perf_counter() - t0)
        # about budget_s seconds of oracle work in all, at least three runs
        if (time.perf_counter() - start >= budget_s and len(times) >= 3) or len(times) >= 50:
            break
    med = statistics.median(times)
    step_s = med * T / Ts
    sample = ("oracle fused expert MLP (gate_up, SiLU*mul, down, combine; binary32 loops) on %s, "
              "median of %d runs of %.2f s" % ("the full step of %d tokens" % T if Ts == T else
                                                 "the first %d of %d tokens, scaled to the step" % (Ts, T),
                                                 len(times), med))
    return {"value": weight_bytes_step / step_s / 1e9, "unit": "GB/s", "cores": threads, "threads": threads,
            "host_cpus": os.cpu_count(), "cpus_available": available_cpus(), "kind": "oracle",
            "cpu_share_cap": CPU_SHARE_THREADS, "sample": sample, "us_per_step": step_s * 1e6}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="deepseek-moe-t4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one elementwise copy of 256 MiB (read 256 MiB, write 256 MiB) before the steps: "
                         "the reference dispatch that scales hardware byte counters to bytes")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import weight_only_int4_amd as w4
    from weight_only_int4_amd import lib as L

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = torch.device("cuda:0")
    spec = workload_spec(args.workload)
    E, k, H, I, T = spec["E"], spec["k"], spec["H"], spec["I"], spec["T"]
    print("[bench] %s" % spec["desc"], file=sys.stderr, flush=True)
    inputs = make_inputs(spec, dev)
    x, ids, tw, c13, s13, c2, s2 = inputs
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    active = np.unique(flat[valid])
    Rv = int(valid.sum())
    fmt = spec.get("fmt", "int4")
    wb13, wb2 = packed_weight_bytes(2 * I, H, fmt), packed_weight_bytes(H, I, fmt)
    weight_bytes_step = len(active) * (wb13 + wb2)

    def u16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    def codes_dev(c):
        return c if isinstance(c, torch.Tensor) else torch.from_numpy(c).to(dev)

    def scales_dev(sc):
        if fmt == "mxfp4":
            return codes_dev(sc)
        return sc.view(torch.int16) if isinstance(sc, torch.Tensor) else u16(sc)

    pack = w4.pack_weights_mxfp4 if fmt == "mxfp4" else w4.pack_weights
    w13 = pack(codes_dev(c13), scales_dev(s13))
    w2 = pack(codes_dev(c2), scales_dev(s2))
    per_copy = w13.packed.numel() + w2.packed.numel()
    ncopies = max(2, math.ceil(ROTATION_BYTES / per_copy) + 1)
    copies = [(w13, w2)]
    for _ in range(ncopies - 1):
        copies.append((w13.rebind(w13.packed.clone()), w2.rebind(w2.packed.clone())))
    xd = u16(x).view(torch.bfloat16)
    idsd = torch.from_numpy(ids).to(dev)
    twd = torch.from_numpy(tw).to(dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    # an expert-parallel share plans for the rows a local expert expects, T*k / (global experts), which is what
    # the caller knows before routing; a whole-model layer uses the call's own estimate T*k/E
    hint = T * k / spec["global_experts"] if "global_experts" in spec else 0.0
    p13, p2 = w4.fused_moe_plans(T, k, w13, w2, expected_rows_per_expert=hint)
    plans = (p13, p2)
    ws = w4.zeroed_workspace(w4.fused_moe_workspace_bytes(T, k, w13, w2, plans), dev)
    print("[bench] plans: gate_up %r, down %r%s; %d active experts, %d local routes; weight pool %d copies x %.1f MB"
          % (p13, p2, " (for %.2f rows per local expert)" % hint if hint else "", len(active), Rv, ncopies,
             per_copy / 1e6), file=sys.stderr, flush=True)

    lib = L.load()
    if args.copy_calibration:
        src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def fused_args(c, stream, events=None):
        a, b = copies[c]
        return (L._ptr(xd), L._ptr(idsd), L._ptr(twd), T, k, a.handle, b.handle, ctypes.byref(p13), ctypes.byref(p2),
                L._ptr(out), L._ptr(ws), ws.numel(), L._stream(stream), events)

    def check(rc):
        if rc:
            raise L.W4A16Error(rc, lib.w4a16_last_error().decode())

    # ---- timed steps: HIP-graph replays of the fused call, one graph per weight copy
    stream = torch.cuda.current_stream()
    for c in range(ncopies):  # eager warm-up of every copy (also initialises the library's launch state)
        check(lib.w4a16_fused_moe_planned(*fused_args(c, stream)))
    torch.cuda.synchronize()
    graphs = []
    for c in range(ncopies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            check(lib.w4a16_fused_moe_planned(*fused_args(c, torch.cuda.current_stream())))
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % ncopies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % ncopies].replay()
    t_enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    ms_per_step = t_total * 1e3 / args.steps
    if t_enqueue > 0.9 * t_total:
        print("[bench] warning: host enqueue (%.1f us/step) is close to the step time" % (t_enqueue * 1e6 / args.steps),
              file=sys.stderr)

    # ---- per-stage GPU time: the same fused call with HIP events between its stages, on the same stream,
    # enqueued behind a GPU-side sleep so that every event pair brackets only GPU work
    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # create the underlying HIP event now
        return e

    NS = len(L.FUSED_STAGES)
    events = [[ev() for _ in range(NS + 1)] for _ in range(args.steps)]
    arrays = [ctypes_array(e) for e in events]  # (pointer, keep-alive array)
    for c in range(ncopies):
        check(lib.w4a16_fused_moe_planned(*fused_args(c, stream, arrays[0][0])))
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * max(0.02, 400e-6 * args.steps)))  # ~clock rate x seconds of host enqueue
    for i in range(args.steps):
        check(lib.w4a16_fused_moe_planned(*fused_args(i % ncopies, stream, arrays[i][0])))
    torch.cuda.synchronize()
    stage = np.array([[events[i][s].elapsed_time(events[i][s + 1]) * 1e3 for s in range(NS)] for i in range(args.steps)])
    gpu_step_us = float(np.mean([events[i][0].elapsed_time(events[i][NS]) * 1e3 for i in range(args.steps)]))
    value = weight_bytes_step / (ms_per_step * 1e-3) / 1e9

    # ---- the dominant kernel alone: its launch as in the fused call (same plan, routing and workspace layout
    # rules), captured back to back in one HIP graph that cycles through the weight copies; HIP events on the
    # launch stream around the replays give the average launch duration without host gaps
    prefill_plan = p13.kernel == L.KERNEL_PREFILL
    route = w4.route_prep(idsd, E, p13.block_m)
    h_out = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    gws = w4.zeroed_workspace(w4.gemm_workspace_bytes(p13, T * k, E, 2 * I), dev)
    reps = max(ncopies, 20 // ncopies * ncopies)
    if prefill_plan:
        reps = ncopies  # launches of milliseconds: one per weight copy is enough
    for c in range(ncopies):
        w4.grouped_gemm_silu(xd, k, copies[c][0], route, p13, out=h_out, ws=gws)
    torch.cuda.synchronize()
    kg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(kg):
        for r in range(reps):
            w4.grouped_gemm_silu(xd, k, copies[r % ncopies][0], route, p13, out=h_out, ws=gws)
    # warm until about 30 ms of these launches have run (the part's clock settles; the first few
    # milliseconds after an idle gap run up to 15% slower), then the median of five timed trials
    t0 = time.perf_counter()
    kg.replay()
    torch.cuda.synchronize()
    first = time.perf_counter() - t0
    for _ in range(min(200, max(1, int(0.03 / max(first, 1e-6))))):
        kg.replay()
    torch.cuda.synchronize()
    n_replay, trials = 5, []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_replay):
            kg.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        trials.append(e0.elapsed_time(e1) * 1e3 / (n_replay * reps))
    gate_up_us = statistics.median(trials)

    # dominant kernel: gate_up grouped GEMM with the SiLU*mul epilogue (decode or prefill kernel by plan).
    # Its roofline is the longer of two minimum times: algorithmic bytes (packed weights of the active experts,
    # x once, h written once, routing read once) at the HBM peak, and algorithmic flops (2 * valid routes * 2I *
    # H) at the dense BF16 matrix peak.
    prefill = p13.kernel == L.KERNEL_PREFILL
    bound, alg_bytes, alg_flops = roofline_bound(spec, p13.block_m)
    mfma_bound = bound == "mfma"
    if mfma_bound:
        achieved = alg_flops / (gate_up_us * 1e-6) / 1e12
    else:
        achieved = alg_bytes / (gate_up_us * 1e-6) / 1e9
    traffic = committed_traffic(spec["name"], "prefill" if prefill else "decode")
    if p13.kernel == L.KERNEL_DECODE and p13.block_m == 16:
        kname = "gemm_decode_reg_kernel<NBW=%d,D=2,act out,%s> (gate_up + silu_mul, k_split %d)" % (
            p13.n_blocks, fmt, p13.k_split)
    else:
        kname = "gemm_%s_kernel<MT=%d,NBW=%d,act out,%s> (gate_up + silu_mul, route blocks of %d rows, " \
                "k_split %d)" % ("decode" if p13.kernel == L.KERNEL_DECODE else "prefill",
                                 (p13.tile_m or p13.block_m) // 16, p13.n_blocks, fmt, p13.block_m, p13.k_split)

    stages = list(L.FUSED_STAGES)
    print("[bench] step %.1f us wall (graph replay), %.1f us GPU events; per stage (us): %s" % (
        ms_per_step * 1e3, gpu_step_us, ", ".join("%s %.1f" % (n, v) for n, v in zip(stages, stage.mean(0)))),
        file=sys.stderr, flush=True)

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s",
        "us_per_call": round(ms_per_step * 1e3, 2), "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": spec["name"], "description": spec["desc"], "experts": E, "top_k": k,
                   "tokens": T, "hidden": H, "intermediate": I, "weight_format": fmt,
                   "active_experts": int(len(active)),
                   "local_routes": Rv, "weight_bytes_per_step": int(weight_bytes_step),
                   "weight_rotation_copies": ncopies, "parallelism": "none (one GPU)"},
        "stages_us": {n: round(float(v), 2) for n, v in zip(stages, stage.mean(0))},
        "one_launch": bool(p13.flags & L.PLAN_ONE_LAUNCH),  # then stages_us.gate_up_silu holds both GEMMs
        "gpu_us_per_step_events": round(gpu_step_us, 2),
        "roofline": ({"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                      "kernel": kname, "flops_per_launch": alg_flops} if mfma_bound else
                     {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kname,
                      "bytes_per_launch": int(alg_bytes)}),
    }
    result["roofline"].update({"avg_launch_us": round(gate_up_us, 2),
                               "timing": "median of 5 trials, each HIP events around %d graph-captured "
                                         "back-to-back launches, after about 30 ms of the same launches"
                                         % (n_replay * reps)})
    # references measured on the same box: a device-to-device copy of 1 GiB (read + write bytes per second), and
    # for a matrix-bound workload a dense BF16 GEMM of the gate_up shape on the valid rows (torch, i.e. the
    # platform's BLAS, no dequantisation, no gather)
    ref = {"copy_gbs": round(measured_copy_gbs(dev), 1)}
    if mfma_bound:
        ref["dense_bf16_gemm_tflops"] = round(measured_dense_gemm_tflops(Rv, 2 * I, H, dev), 1)
        ref["kernel_vs_dense_gemm"] = round(achieved / ref["dense_bf16_gemm_tflops"], 4)
    else:
        ref["kernel_vs_copy"] = round(achieved / ref["copy_gbs"], 4)
    result["roofline"]["measured_references"] = ref
    if p13.kernel == L.KERNEL_DECODE and p13.block_m == 16 and T * k <= 4096:
        # inside the fused step this gate_up routes its rows itself (no routing launch): its stage time from the
        # per-stage events, a launch gap included, against the same roofline
        st = float(stage.mean(0)[stages.index("gate_up_silu")])
        ach = (alg_flops / (st * 1e-6) / 1e12) if mfma_bound else (alg_bytes / (st * 1e-6) / 1e9)
        result["roofline"]["step_form"] = {
            "kernel": kname.replace("act out,", "act out, routes its rows in-kernel,"),
            "stage_us": round(st, 2), "achieved": round(ach, 1),
            "frac": round(ach / (MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS), 4),
            "timing": "mean over the timed steps of HIP events around the gate_up stage of eager fused calls "
                      "(includes the gap between launches)"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, inputs, weight_bytes_step, args.cpu_budget)
    print(json.dumps(result), flush=True)


def _event_median_us(fn, reps=10, trials=5):
    import torch

    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    return statistics.median(ts)


def measured_copy_gbs(dev, nbytes=1 << 30):
    """Device-to-device copy bandwidth on this machine (bytes read plus bytes written per second, GB/s)."""
    import torch

    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    us = _event_median_us(lambda: dst.copy_(src))
    del src, dst
    return 2 * nbytes / (us * 1e-6) / 1e9


def measured_dense_gemm_tflops(M, N, K, dev):
    """A dense BF16 GEMM [M,K] x [K,N] through torch on this machine (TFLOP/s): the matrix-core rate the platform's
    BLAS reaches on the same shape with nothing to dequantise or gather."""
    import torch

    a = torch.randn((M, K), device=dev).to(torch.bfloat16)
    b = torch.randn((K, N), device=dev).to(torch.bfloat16)  # contiguous, not a transposed view
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    us = _event_median_us(lambda: torch.mm(a, b, out=c))
    del a, b, c
    return 2.0 * M * N * K / (us * 1e-6) / 1e12


def ctypes_array(evs):
    import ctypes

    arr = (ctypes.c_void_p * len(evs))(*[ctypes.c_void_p(e.cuda_event) for e in evs])
    return ctypes.cast(arr, ctypes.c_void_p), arr


if __name__ == "__main__":
    main()
