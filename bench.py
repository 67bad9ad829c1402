#!/usr/bin/env python3
"""Benchmark of the routed NVFP4 MoE layer on one MI355X.

One step = one layer: moe_route_bucket + moe_ffn_nvfp4 over one batch of synthetic input that is
already resident in HBM. The default workload is the verify chunk (E=512 experts, hidden 2560,
ff 640, top-10, 6 tokens = 60 routed slots, union of 60 distinct experts), the decode shape the
moe_union_probe page prices. Consecutive steps use routing over disjoint expert windows so that
every step streams its experts' weights from HBM, not from the 256 MB Infinity Cache.

Prints one JSON line: value = unique-expert weight bytes per second (decode workloads) or useful
TFLOP/s (prefill workloads), the dominant kernel's roofline from HIP events recorded around its
launches, and the fp64 oracle timed on a bounded sample on the host cores.
"""
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

METRIC = "routed-MoE layer µs + HBM GB/s (% of 8 TB/s) at T=1..128; TFLOP/s at T=4096"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense MFMA, f16 and bf16 alike (the GEMMs run f16)
COPY_BYTES = 1 << 30

# HBM traffic of the dominant kernel, per launch, from two rocprofv3 --pmc passes over
# `bench.py --steps 20 --warmup 5 --no-cpu-baseline` (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch, mean over the dispatches). Each counter is scaled by what it reads for
# `bench.py --copy-calib` (a 1 GiB copy): FETCH_SIZE read 524301 KiB for 1048576 KiB moved, so x2.0;
# WRITE_SIZE read 1048576 KiB, so x1.0. Keyed by the SHA-256 of the kernel's sources: once they
# change, the entry no longer applies and traffic is reported as null until measured again.
FETCH_SCALE = 1048576.0 / 524301.2
WRITE_SCALE = 1.0
TRAFFIC = {
    ("gu_decode_kernel", "verify_chunk", 6, 60): {
        "sources": ["routed_moe_expert_amd/csrc/ffn_decode.hip",
                    "routed_moe_expert_amd/csrc/moe_internal.h"],
        "sha256": "e7a723f1467c7a4b04c79c0b729cb65f901f1608de4f57ce3edf8f7762b65dda",
        "fetch_kib": 54326.5, "write_kib": 169.0,
    },
    # (`bench.py --workload full_prefill --steps 4 --warmup 1 --no-cpu-baseline`)
    ("gemm_kernel<false>", "full_prefill", 4096, None): {
        "sources": ["routed_moe_expert_amd/csrc/ffn_prefill.hip",
                    "routed_moe_expert_amd/csrc/moe_internal.h"],
        "sha256": "faa674bc3b45a1d3ac93801fa75855425e55c45c2b9b495e671e2cc1fbfec7a8",
        "fetch_kib": 1339114.5, "write_kib": 175615.4,
    },
}


def measured_traffic(kname, workload, T, U):
    """Calibrated HBM bytes per launch of `kname`, or None if not measured for these sources."""
    import hashlib
    ent = TRAFFIC.get((kname, workload, T, U))
    if ent is None:
        return None
    h = hashlib.sha256()
    for f in ent["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != ent["sha256"]:
        return None
    fetch = ent["fetch_kib"] * 1024 * FETCH_SCALE
    write = ent["write_kib"] * 1024 * WRITE_SCALE
    return {"bytes": fetch + write, "fetch_bytes": fetch, "write_bytes": write}


def _hip():
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="verify_chunk",
                    choices=["verify_chunk", "tiny_decode", "e256_plateau", "skewed_prefill",
                             "full_prefill", "shared_expert", "router"])
    ap.add_argument("--E", type=int, default=288, help="experts (router workload)")
    ap.add_argument("--k", type=int, default=8, help="top-k (router workload)")
    ap.add_argument("--T", type=int, default=None, help="tokens (workload default if unset)")
    ap.add_argument("--U", type=int, default=60, help="union size for verify_chunk")
    ap.add_argument("--virtual", type=int, default=0,
                    help="shared_expert: virtual experts over its one weight copy (0: T/16)")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--warm", action="store_true", help="reuse one routing (cache-warm numbers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scale for HBM byte counters)")
    return ap.parse_args()


def copy_calibration(torch):
    """A plain copy of known size: it reads and writes COPY_BYTES per launch, so what a
    FETCH_SIZE / WRITE_SIZE counter reads for it converts that counter to bytes."""
    src = torch.full((COPY_BYTES,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": COPY_BYTES, "launches": 5}), flush=True)


DEFAULT_T = {"verify_chunk": 6, "tiny_decode": 1, "e256_plateau": 128, "skewed_prefill": 4096,
             "full_prefill": 4096, "shared_expert": 128}


def build_inputs(args, torch, gen, moe):
    """Host generation + upload. Returns (steps callables data, description dict)."""
    import numpy as np

    name = args.workload
    w = gen.WORKLOADS[name]
    E, H, F, k, seed = w["E"], w["H"], w["F"], w["k"], w["seed"]
    T = args.T or DEFAULT_T[name]
    U = None
    copies = 1
    virtual = 0
    if name == "verify_chunk":
        U = args.U
        variants = [gen.route_union_rotated(seed, T, k, E, U, v)
                    for v in range(1 if args.warm else math.ceil(2 * E / U) + 1)]
    elif name == "tiny_decode":
        U = k
        copies = 1 if args.warm else 3          # 3 bank copies x disjoint windows > 2 x 256 MB
        variants = [gen.route_union_rotated(seed, T, k, E, k, v)
                    for v in range(1 if args.warm else E // k)]
    elif name == "shared_expert":
        # the one expert as G virtual experts (pointer tables onto its one copy), tokens dealt
        # round-robin: the same dense SwiGLU with G times the work items
        virtual = args.virtual or max(1, math.ceil(T / 16))
        variants = [gen.shared_virtual_routing(T, virtual)[0]]
    else:
        variants = [gen.make_routing(name, T)[0]]
    banks = gen.make_banks(E, H, F, w["fused"], seed)
    x = gen.bf16_normal(seed, (T, H))
    wts = gen.make_routing(name, T)[1] if name == "shared_expert" else gen.router_weights(seed, T, k)

    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                   else np.ascontiguousarray(a)).to(dev)
    rbh, rbf = H // 64 * 36, F // 64 * 36
    bank_sets = []
    for c in range(copies):
        if w["fused"]:
            gu = t(banks["gate_up"])
            gate, up = moe.bank(gu, 2 * F * rbh), moe.bank(gu, 2 * F * rbh, F * rbh)
            keep = [gu]
        else:
            g_, u_ = t(banks["gate"]), t(banks["up"])
            gate, up = moe.bank(g_, F * rbh), moe.bank(u_, F * rbh)
            keep = [g_, u_]
        d_ = t(banks["down"])
        down = moe.bank(d_, H * rbf)
        keep.append(d_)
        if virtual:
            tabs = [torch.full((virtual,), b.base, dtype=torch.int64, device=dev)
                    for b in (gate, up, down)]
            gate, up, down = (moe.bank(None, 0, experts=tb) for tb in tabs)
            keep += tabs
        bank_sets.append((gate, up, down, keep))
    del banks
    ids_dev = [t(v.reshape(-1).astype(np.int32)) for v in variants]
    uniq = [1] if virtual else [int(np.unique(v).size) for v in variants]
    out = dict(name=name, E=virtual or E, H=H, F=F, k=k, T=T, U=U, copies=copies,
               variants=variants, ids=ids_dev, uniq=uniq, x=t(x), w=t(wts.reshape(-1)),
               bank_sets=bank_sets, host=dict(x=x, w=wts), virtual=virtual)
    if virtual:   # the oracle takes the plain one-expert form
        out.update(oracle_E=E, oracle_ids=np.zeros((T, 1), dtype=np.int32))
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the routed layer here is one GPU's share; multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calib:
        copy_calibration(torch)
        return

    import gen
    import routed_moe_expert_amd as moe

    torch.cuda.set_device(0)
    if args.workload == "router":
        bench_router(args, torch, gen, moe)
        return
    D = build_inputs(args, torch, gen, moe)
    E, H, F, k, T = D["E"], D["H"], D["F"], D["k"], D["T"]
    P = T * k
    path = {"auto": moe.MOE_PATH_AUTO, "decode": moe.MOE_PATH_DECODE,
            "prefill": moe.MOE_PATH_PREFILL}[args.path]
    eff_path = path if path else (moe.MOE_PATH_DECODE if T <= 128 else moe.MOE_PATH_PREFILL)
    decode = eff_path == moe.MOE_PATH_DECODE

    dev = torch.device("cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pair_ids = torch.empty(P, dtype=torch.int32, device=dev)
    active = torch.empty(E, dtype=torch.int32, device=dev)
    counts = torch.empty(2, dtype=torch.int32, device=dev)
    bws = moe.moe_route_bucket_ws(T, k, E)
    bucket_ws = torch.empty(max(bws, 1), dtype=torch.uint8, device=dev)
    fws = moe.moe_ffn_nvfp4_ws(T, k, E, H, F)
    ws = torch.empty(fws, dtype=torch.uint8, device=dev)
    y = torch.empty(T, H, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    nv, nc = len(D["ids"]), D["copies"]

    def step(i):
        ids = D["ids"][i % nv]
        gate, up, down, _ = D["bank_sets"][(i // nv) % nc if nc > 1 else 0]
        moe.moe_route_bucket(ids, T, k, E, 0, offsets, pair_ids, active, counts, bucket_ws, bws,
                             stream=sh)
        moe.moe_ffn_nvfp4(D["x"], D["w"], offsets, pair_ids, active, counts, gate, up, down, T,
                          k, E, H, F, y, path, ws, fws, stream=sh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, an event before each step for per-layer times
    K = args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        evs[i].record(stream)
        step(args.warmup + i)
    evs[K].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]
    ms_per_step = evs[0].elapsed_time(evs[K]) / K

    # dominant kernel: HIP events recorded by the library around each of its launches, over a
    # second pass of the same K steps
    hip = _hip()
    kid = moe.MOE_KERNEL_GU_DECODE if decode else moe.MOE_KERNEL_GU_PREFILL
    kname = "gu_decode_kernel" if decode else "gemm_kernel<false>"   # gate/up + SiLU
    starts, stops = [], []
    for _ in range(K):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        hip.hipEventCreate(ctypes.byref(a))
        hip.hipEventCreate(ctypes.byref(b))
        starts.append(a.value)
        stops.append(b.value)
    torch.cuda.synchronize()
    moe.moe_profile_kernel(kid, starts, stops)
    for i in range(K):
        step(args.warmup + i)
    torch.cuda.synchronize()
    n_rec = moe.moe_profile_count()
    moe.moe_profile_kernel(moe.MOE_KERNEL_NONE, [], [])
    kms = []
    for i in range(n_rec):
        f = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(starts[i]), ctypes.c_void_p(stops[i]))
        kms.append(f.value)
    for a, b in zip(starts, stops):
        hip.hipEventDestroy(ctypes.c_void_p(a))
        hip.hipEventDestroy(ctypes.c_void_p(b))
    k_avg_s = (sum(kms) / len(kms)) * 1e-3 if kms else float("nan")

    rbh, rbf = H // 64 * 36, F // 64 * 36
    per_expert = 2 * F * rbh + H * rbf
    uniq = statistics.mean(D["uniq"])
    unique_bytes = uniq * per_expert
    useful_flops = 6.0 * P * H * F
    s = ms_per_step * 1e-3
    med = statistics.median(per)
    layer = {"us_mean": ms_per_step * 1e3, "us_min": min(per) * 1e3, "us_median": med * 1e3,
             "spread": (max(per) - min(per)) / med if med > 0 else None}
    if decode:
        value, unit = unique_bytes / s / 1e9, "GB/s"
        gu_bytes = uniq * 2 * F * rbh + T * H * 2 + P * F * 4
        roof = {"bound": "hbm", "kernel": kname, "achieved": gu_bytes / k_avg_s / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "bytes_per_launch": gu_bytes, "avg_launch_us": k_avg_s * 1e6, "launches": len(kms)}
        roof["frac"] = roof["achieved"] / roof["peak"]
    else:
        value, unit = useful_flops / s / 1e12, "TFLOP/s"
        gu_flops = 4.0 * P * H * F
        roof = {"bound": "mfma", "kernel": kname, "achieved": gu_flops / k_avg_s / 1e12,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "flops_per_launch": gu_flops,
                "avg_launch_us": k_avg_s * 1e6, "launches": len(kms)}
        roof["frac"] = roof["achieved"] / roof["peak"]
    tr = measured_traffic(kname, D["name"], T, D["U"] if D["name"] == "verify_chunk" else None)
    roof["traffic"] = tr["bytes"] if tr else None
    if tr:
        # prefill gate/up: the unique experts' gate and up weights, x (f16) once, h hi + lo
        alg = gu_bytes if decode else uniq * 2 * F * rbh + T * H * 2 + P * F * 4
        roof["traffic_detail"] = tr
        roof["traffic_over_algorithmic"] = tr["bytes"] / alg

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, D, gen, unit, per_expert)

    # weights cycled through by the steps: a cyclic sweep larger than the 256 MB Infinity Cache
    # misses it; a smaller one can stay resident
    cycled = min(E, sum(D["uniq"])) * per_expert * D["copies"]
    if args.warm:
        hbm_note = "warm (one routing reused)"
    elif cycled < 256e6:
        hbm_note = (f"cache-resident: {cycled / 1e6:.1f} MB of weights in rotation, under the "
                    "256 MB Infinity Cache")
    else:
        hbm_note = (f"cold ({len(D['ids'])} routings over disjoint expert windows x "
                    f"{D['copies']} bank copies, {cycled / 1e6:.0f} MB of weights in rotation)")
    wl = D["name"]
    desc = {"verify_chunk": f"verify chunk: E={E} H={H} F={F} top-{k} T={T}, union U={D['U']}",
            "tiny_decode": f"tiny decode: E={E} H={H} F={F} top-{k} T={T}",
            "e256_plateau": f"rank-local E256 plateau: E={E} H={H} F={F} top-{k} T={T}",
            "skewed_prefill": f"skewed prefill: E={E} H={H} F={F} top-{k} T={T}",
            "full_prefill": f"full-width prefill: E={E} H={H} F={F} top-{k} T={T}",
            "shared_expert": f"shared expert (dense SwiGLU, every token): H={H} F={F} T={T}, "
                             f"as {D['virtual']} virtual experts over its one weight copy"}[wl]
    out = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": desc, "E": E, "H": H, "F": F, "top_k": k, "T": T,
                   "path": "decode" if decode else "prefill",
                   "hbm": hbm_note},
        "layer": layer,
        "unique_expert_bytes": unique_bytes,
        "per_slot_bytes": P * per_expert,   # what a per-slot path would stream
        "hbm_frac_unique": (unique_bytes / s / 1e9) / HBM_PEAK_GBS,
        "useful_tflops": useful_flops / s / 1e12,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)


def kernel_times_ms(moe, kid, K, step):
    """Average of the library's HIP-event times of kernel `kid` over K more calls of step(i)."""
    import torch
    hip = _hip()
    starts, stops = [], []
    for _ in range(K):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        hip.hipEventCreate(ctypes.byref(a))
        hip.hipEventCreate(ctypes.byref(b))
        starts.append(a.value)
        stops.append(b.value)
    torch.cuda.synchronize()
    moe.moe_profile_kernel(kid, starts, stops)
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    n_rec = moe.moe_profile_count()
    moe.moe_profile_kernel(moe.MOE_KERNEL_NONE, [], [])
    kms = []
    for i in range(n_rec):
        f = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(starts[i]), ctypes.c_void_p(stops[i]))
        kms.append(f.value)
    for a, b in zip(starts, stops):
        hip.hipEventDestroy(ctypes.c_void_p(a))
        hip.hipEventDestroy(ctypes.c_void_p(b))
    return (sum(kms) / len(kms) if kms else float("nan")), len(kms)


def bench_router(args, torch, gen, moe):
    """The router step alone (moe_router_topk): fp32 logits [T, E] -> top-k ids and softmax
    weights. One step = one call over one logits batch; consecutive steps read different copies
    so that more than 2 x 256 MB cycle through (the logits come from HBM, not the Infinity Cache,
    where a batch is large enough for that to matter)."""
    import numpy as np
    import oracle

    T, E, k = args.T or 4096, args.E, args.k
    logits = gen.router_logits(11, T, E)
    lb = T * E * 4
    copies = max(1, min(128, math.ceil(512e6 / lb)))
    dev = torch.device("cuda")
    base = torch.from_numpy(logits).to(dev)
    lg = [base.clone() for _ in range(copies)]
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream().cuda_stream

    def step(i):
        moe.moe_router_topk(lg[i % copies], T, E, k, ids, w, stream=sh)

    for i in range(args.warmup):
        step(i)
    K = args.steps
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / K
    k_ms, n_k = kernel_times_ms(moe, moe.MOE_KERNEL_ROUTER, K, step)
    nbytes = lb + T * k * 8
    s = ms_per_step * 1e-3
    roof = {"bound": "hbm", "kernel": "router_topk_kernel", "achieved": nbytes / (k_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_launch": nbytes,
            "avg_launch_us": k_ms * 1e3, "launches": n_k, "traffic": None}
    roof["frac"] = roof["achieved"] / roof["peak"]
    cpu = None
    if not args.no_cpu_baseline:
        n = min(T, 4096)
        t1 = time.perf_counter()
        reps = 0
        while True:
            oracle.router_topk(logits[:n], k)
            reps += 1
            el = time.perf_counter() - t1
            if el >= min(args.cpu_seconds, 10.0):
                break
        sec = el / reps * T / n
        cpu = {"value": nbytes / sec / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} of the {T} tokens per repetition, scaled to the batch",
               "seconds_per_batch": sec, "reps": reps}
    out = {
        "metric": "router step µs + GB/s of logits read and ids/weights written",
        "value": nbytes / s / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"router top-{k}: E={E} T={T}, N(0,1) fp32 logits", "E": E,
                   "top_k": k, "T": T, "hbm": f"{copies} logits copies in rotation"},
        "step_us": ms_per_step * 1e3,
        "roofline": roof,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(args, D, gen, unit, per_expert):
    """The fp64 oracle (union form) timed on the host cores on a bounded sample of the same
    workload, scaled to the metric's unit."""
    import numpy as np

    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or min(os.cpu_count() or 1, 16)
    name = D["name"]
    w = gen.WORKLOADS[name]
    E, H, F, k, T = D.get("oracle_E", D["E"]), D["H"], D["F"], D["k"], D["T"]
    banks = gen.make_banks(E, H, F, w["fused"], w["seed"])
    ids = D.get("oracle_ids", D["variants"][0])
    if T * k <= 160 or name != "skewed_prefill" and name != "full_prefill":
        tok = None
        sample = f"whole layer (all {T} tokens, {T * k} routed slots), union form"
    else:
        tok = np.arange(8)
        sample = "8 of the layer's tokens (64 routed slots), per-slot form"
    case = dict(E=E, H=H, F=F, k=k, T=T, ids=ids, w=D["host"]["w"], x=D["host"]["x"], **banks)
    t0 = time.perf_counter()
    reps = 0
    while True:
        if tok is None:
            oracle.ffn_union(case, threads=threads)
        else:
            oracle.ffn_per_slot(case, tokens=tok, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or el * (reps + 1) / reps > 30.0:
            break
    sec = el / reps

    def rate(sec_, ids_, n_pairs):
        if unit == "GB/s":
            return len(np.unique(ids_)) * per_expert / sec_ / 1e9
        return 6.0 * n_pairs * H * F / sec_ / 1e12

    v = rate(sec, ids, T * k if tok is None else len(tok) * k)
    # one thread, on the first token's slots (same form as above), once
    t1 = time.perf_counter()
    if tok is None:
        one = dict(case, T=1, ids=ids[:1], w=D["host"]["w"][:1], x=D["host"]["x"][:1])
        oracle.ffn_union(one, threads=1)
    else:
        oracle.ffn_per_slot(case, tokens=np.arange(1), threads=1)
    sec1 = time.perf_counter() - t1
    single = {"value": rate(sec1, ids[:1], k), "cores": 1,
              "sample": f"the first token ({k} routed slots), "
                        f"{'union' if tok is None else 'per-slot'} form, once",
              "seconds_per_sample": sec1}
    return {"value": v, "unit": unit, "cores": threads, "kind": "oracle", "sample": sample,
            "seconds_per_sample": sec, "reps": reps, "single_thread": single}


if __name__ == "__main__":
    main()
