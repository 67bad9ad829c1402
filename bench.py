#!/usr/bin/env python3
"""Benchmark of the routed NVFP4 MoE layer on one MI355X.

One step = one layer over one batch of synthetic input that is already resident in HBM: one call
of moe_layer_nvfp4 (routed ids -> y; the same as moe_route_bucket + moe_ffn_nvfp4, which is timed
beside it as `two_call_layer_us`). The headline workload is the verify chunk (E=512 experts, hidden 2560,
ff 640, top-10, 6 tokens = 60 routed slots, union of 60 distinct experts), the decode shape the
moe_union_probe page prices. Consecutive steps use routing over disjoint expert windows so that
every step streams its experts' weights from HBM, not from the 256 MB Infinity Cache.

Every timed region is queued behind a bounded sleep kernel, so all of its launches are enqueued
before the GPU reaches the first one: the HIP events then time the GPU alone, not the host's
launch rate. The layer time is the mean over K back-to-back layers between two events; a second
pass with an event between every two layers gives the per-step distribution (those events are
queue packets of their own and add about 3 us per decode layer).

Where a layer runs the grouped-GEMM path, its banks also carry their K-step-packed copies
(moe_kpack, written once before any timing, as a model would at load time), which the GEMMs read;
`--no-kpack` times the GEMMs on the row-major banks. The decode path reads the row-major banks.

Prints one JSON line: value = unique-expert weight bytes per second (decode workloads) or useful
TFLOP/s (prefill workloads), the dominant kernel's roofline from HIP events recorded around its
launches, the fp64 oracle timed on a bounded sample on the host cores, and `rows`: the same
measurement for every configuration of the layer (tiny decode, verify chunk at three union
sizes, the rank-local E256 plateau at five token counts, the skewed prefill at three, the
full-width prefill).
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
F16_PEAK_TFLOPS = 2500.0     # MI355X dense MFMA, f16 and bf16 alike (the GEMMs run f16)
COPY_BYTES = 1 << 30

# HBM traffic of the dominant kernel, per launch, from two rocprofv3 --pmc passes over
# `bench.py --rows none --no-cpu-baseline --layer-only --steps 20 --warmup 5` (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, mean over the dispatches). Each counter is scaled by what it reads
# for `bench.py --copy-calib` (a 1 GiB copy): FETCH_SIZE read 524302 KiB for 1048576 KiB moved,
# so x2.0; WRITE_SIZE read 1048576 KiB, so x1.0. Keyed by the SHA-256 of the kernel's sources: once
# they change, the entry no longer applies and traffic is reported as null until measured again.
FETCH_SCALE = 1048576.0 / 524302.3
WRITE_SCALE = 1.0
TRAFFIC = {
    ("gu_decode_kernel", "verify_chunk", 6, 60): {
        "sources": ["routed_moe_expert_amd/csrc/ffn_decode.hip",
                    "routed_moe_expert_amd/csrc/moe_internal.h"],
        "sha256": "e29566e8f962d11c3ad900dba8522c109ae073e68dece055e66e21665f6ea2e4",
        "fetch_kib": 54367.0, "write_kib": 168.2,
    },
}

# every configuration of the layer: (workload, tokens, union size for the verify chunk)
ROWS = [("tiny_decode", 1, None), ("verify_chunk", 6, 10), ("verify_chunk", 6, 30),
        ("verify_chunk", 6, 60), ("e256_plateau", 16, None), ("e256_plateau", 32, None),
        ("e256_plateau", 64, None), ("e256_plateau", 80, None), ("e256_plateau", 128, None),
        ("skewed_prefill", 512, None), ("skewed_prefill", 2048, None),
        ("skewed_prefill", 4096, None), ("full_prefill", 4096, None)]

DEFAULT_T = {"verify_chunk": 6, "tiny_decode": 1, "e256_plateau": 128, "skewed_prefill": 4096,
             "full_prefill": 4096, "shared_expert": 128}


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
    ap.add_argument("--rows", default="all", choices=["all", "none"],
                    help="also time every configuration of the layer (the `rows` key)")
    ap.add_argument("--E", type=int, default=288, help="experts (router workload)")
    ap.add_argument("--k", type=int, default=8, help="top-k (router workload)")
    ap.add_argument("--T", type=int, default=None, help="tokens (workload default if unset)")
    ap.add_argument("--U", type=int, default=60, help="union size for verify_chunk")
    ap.add_argument("--virtual", type=int, default=0,
                    help="shared_expert: route it as G caller-side virtual experts over its one "
                         "weight copy (0: the one expert, E=1)")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--no-kpack", action="store_true",
                    help="GEMM path from the row-major banks (default: from K-step-packed copies)")
    ap.add_argument("--warm", action="store_true", help="reuse one routing (cache-warm numbers)")
    ap.add_argument("--layer-only", action="store_true",
                    help="time only the one-call layer (not also the two calls), e.g. under a profiler")
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


# ----------------------------------------------------------------------------------- timing

class Queue:
    """Times GPU work free of host launch overhead: a bounded sleep kernel is queued first, long
    enough for the host to enqueue the whole timed region behind it."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        # GPU time per sleep cycle, measured once
        a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        torch.cuda.synchronize()
        a.record(self.stream)
        torch.cuda._sleep(2_000_000)
        b.record(self.stream)
        torch.cuda.synchronize()
        self.ms_per_cycle = max(a.elapsed_time(b), 1e-3) / 2_000_000

    def run(self, enqueue, host_ms_hint):
        """Sleep, then enqueue(); returns (host enqueue ms, sleep ms, whether the sleep outlasted
        the enqueue). host_ms_hint: expected host time to enqueue."""
        torch = self.torch
        want_ms = min(max(3.0 * host_ms_hint + 2.0, 5.0), 2000.0)
        cycles = int(want_ms / self.ms_per_cycle)
        s0, s1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        torch.cuda.synchronize()
        s0.record(self.stream)
        torch.cuda._sleep(cycles)
        s1.record(self.stream)
        t0 = time.perf_counter()
        enqueue()
        host_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        sleep_ms = s0.elapsed_time(s1)
        return host_ms, sleep_ms, host_ms < sleep_ms


def time_steps(q, step, K, first):
    """GPU time of K steps (step(first + i)), queued behind a sleep, twice: once with an event
    between every two steps (the per-step distribution), once with events only around the K
    steps (the mean per step: each event is a packet of its own in the queue, and one between
    every two steps measured about 3 us more per decode layer). Returns (per-step ms, mean ms
    per step over the span, queue info)."""
    torch = q.torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    step(first)
    torch.cuda.synchronize()
    hint = (time.perf_counter() - t0) * 1e3 * K

    def enqueue():
        for i in range(K):
            evs[i].record(q.stream)
            step(first + i)
        evs[K].record(q.stream)

    host_ms, sleep_ms, ahead = q.run(enqueue, hint)
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]

    def enqueue_span():
        evs[0].record(q.stream)
        for i in range(K):
            step(first + i)
        evs[K].record(q.stream)

    host2, sleep2, ahead2 = q.run(enqueue_span, hint)
    span = evs[0].elapsed_time(evs[K]) / K
    return per, span, {"host_enqueue_ms": host_ms, "sleep_ms": sleep_ms, "queued_ahead": ahead,
                       "span_queued_ahead": ahead2}


def kernel_avg_ms(q, moe, kid, step, K, first):
    """Average GPU ms of kernel `kid` over K steps: HIP events the library records around each
    of its launches (on the launch stream), queued behind a sleep."""
    hip = _hip()
    starts, stops = [], []
    for _ in range(K):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        hip.hipEventCreate(ctypes.byref(a))
        hip.hipEventCreate(ctypes.byref(b))
        starts.append(a.value)
        stops.append(b.value)

    def enqueue():
        moe.moe_profile_kernel(kid, starts, stops)
        for i in range(K):
            step(first + i)

    t0 = time.perf_counter()
    step(first)
    q.torch.cuda.synchronize()
    q.run(enqueue, (time.perf_counter() - t0) * 1e3 * K)
    n_rec = moe.moe_profile_count()
    moe.moe_profile_kernel(moe.MOE_KERNEL_NONE, [], [])
    kms = []
    for i in range(n_rec):
        f = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(starts[i]),
                                ctypes.c_void_p(stops[i]))
        kms.append(f.value)
    for a, b in zip(starts, stops):
        hip.hipEventDestroy(ctypes.c_void_p(a))
        hip.hipEventDestroy(ctypes.c_void_p(b))
    return (sum(kms) / len(kms) if kms else float("nan")), len(kms)


# ----------------------------------------------------------------------------------- inputs

def make_banks_host(gen, name):
    w = gen.WORKLOADS[name]
    return gen.make_banks(w["E"], w["H"], w["F"], w["fused"], w["seed"])


def uses_gemm(gen, moe, name, T, path, args):
    """Whether the layer runs the GEMM path (and so reads K-step-packed copies unless --no-kpack);
    the packed copies are made only then."""
    if args.no_kpack or name == "shared_expert":
        return False
    w = gen.WORKLOADS[name]
    p = path if path != moe.MOE_PATH_AUTO else moe.moe_auto_path(T, w["k"], w["E"], w["H"],
                                                                 w["F"])
    return p == moe.MOE_PATH_PREFILL


def build_inputs(name, T, U, warm, virtual, torch, gen, moe, host_banks=None, kpack=False):
    """Host generation + upload of one workload at T tokens. kpack: the banks also carry their
    K-step-packed copies (moe_kpack, written here, before any timing), which the GEMM path reads."""
    import numpy as np

    w = gen.WORKLOADS[name]
    E, H, F, k, seed = w["E"], w["H"], w["F"], w["k"], w["seed"]
    copies = 1
    if name == "verify_chunk":
        variants = [gen.route_union_rotated(seed, T, k, E, U, v)
                    for v in range(1 if warm else math.ceil(2 * E / U) + 1)]
    elif name == "tiny_decode":
        U = k
        copies = 1 if warm else 3          # 3 bank copies x disjoint windows > 2 x 256 MB
        variants = [gen.route_union_rotated(seed, T, k, E, k, v)
                    for v in range(1 if warm else E // k)]
    elif name == "shared_expert":
        # the one expert (E = 1), or with virtual = G as G virtual experts (pointer tables onto
        # its one copy, tokens dealt round-robin): the same dense SwiGLU
        variants = [gen.shared_virtual_routing(T, virtual)[0] if virtual
                    else np.zeros((T, 1), dtype=np.int32)]
    else:
        variants = [gen.make_routing(name, T)[0]]
        virtual = 0
    if name != "shared_expert":
        virtual = 0
    banks = host_banks if host_banks is not None else make_banks_host(gen, name)
    x = gen.bf16_normal(seed, (T, H))
    wts = gen.make_routing(name, T)[1] if name == "shared_expert" else gen.router_weights(seed, T, k)

    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                   else np.ascontiguousarray(a)).to(dev)
    rbh, rbf = H // 64 * 36, F // 64 * 36
    bank_sets = []
    for _ in range(copies):
        if w["fused"]:
            gu = t(banks["gate_up"])
            gate, up = moe.bank(gu, 2 * F * rbh), moe.bank(gu, 2 * F * rbh, F * rbh)
        else:
            g_, u_ = t(banks["gate"]), t(banks["up"])
            gate, up = moe.bank(g_, F * rbh), moe.bank(u_, F * rbh)
        down = moe.bank(t(banks["down"]), H * rbf)
        if virtual:
            strided = (gate, up, down)
            tabs = [torch.full((virtual,), b.base, dtype=torch.int64, device=dev)
                    for b in strided]
            gate, up, down = (moe.bank(None, 0, experts=tb) for tb in tabs)
            gate._keep += (strided,)   # the tables point into these banks' tensors
        if kpack:
            gate, up, down = (moe.with_kpack(gate, E, F, H), moe.with_kpack(up, E, F, H),
                              moe.with_kpack(down, E, H, F))
            torch.cuda.synchronize()
        bank_sets.append((gate, up, down))
    ids_dev = [t(v.reshape(-1).astype(np.int32)) for v in variants]
    uniq = [1] if virtual else [int(np.unique(v).size) for v in variants]
    out = dict(name=name, E=virtual or E, H=H, F=F, k=k, T=T, U=U, copies=copies,
               variants=variants, ids=ids_dev, uniq=uniq, x=t(x), w=t(wts.reshape(-1)),
               bank_sets=bank_sets, host=dict(x=x, w=wts, banks=banks), virtual=virtual,
               kpack=kpack)
    if virtual:   # the oracle takes the plain one-expert form
        out.update(oracle_E=E, oracle_ids=np.zeros((T, 1), dtype=np.int32))
    return out


class Layer:
    """Device buffers and the step function for one workload."""

    def __init__(self, D, path, torch, moe, fused=True):
        E, H, k, T = D["E"], D["H"], D["k"], D["T"]
        P = T * k
        dev = torch.device("cuda")
        self.D, self.moe = D, moe
        self.path = path
        self.fused = fused
        self.lws = moe.moe_layer_nvfp4_ws(T, k, E, H, D["F"])
        self.layer_ws = torch.empty(self.lws if fused else 1, dtype=torch.uint8, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.pair_ids = torch.empty(P, dtype=torch.int32, device=dev)
        self.active = torch.empty(E, dtype=torch.int32, device=dev)
        self.counts = torch.empty(2, dtype=torch.int32, device=dev)
        self.bws = moe.moe_route_bucket_ws(T, k, E)
        self.bucket_ws = torch.empty(max(self.bws, 1), dtype=torch.uint8, device=dev)
        self.fws = moe.moe_ffn_nvfp4_ws(T, k, E, H, D["F"])
        self.ws = torch.empty(self.fws, dtype=torch.uint8, device=dev)
        self.y = torch.empty(T, H, dtype=torch.float32, device=dev)
        self.sh = torch.cuda.current_stream().cuda_stream

    def step(self, i):
        D, moe = self.D, self.moe
        nv, nc = len(D["ids"]), D["copies"]
        ids = D["ids"][i % nv]
        gate, up, down = D["bank_sets"][(i // nv) % nc if nc > 1 else 0]
        E, H, F, k, T = D["E"], D["H"], D["F"], D["k"], D["T"]
        if self.fused:   # one call: routed ids -> y
            moe.moe_layer_nvfp4(ids, 0, D["x"], D["w"], gate, up, down, T, k, E, H, F, self.y,
                                self.path, self.layer_ws, self.lws, stream=self.sh)
            return
        moe.moe_route_bucket(ids, T, k, E, 0, self.offsets, self.pair_ids, self.active,
                             self.counts, self.bucket_ws, self.bws, stream=self.sh)
        moe.moe_ffn_nvfp4(D["x"], D["w"], self.offsets, self.pair_ids, self.active, self.counts,
                          gate, up, down, T, k, E, H, F, self.y, self.path, self.ws, self.fws,
                          stream=self.sh)


def kernel_table(D, decode):
    """(id, name, amount per launch, unit, peak) of the two big kernels of the path: algorithmic
    HBM bytes for the decode kernels, useful flops for the GEMMs."""
    import routed_moe_expert_amd as moe
    E, H, F, k, T = D["E"], D["H"], D["F"], D["k"], D["T"]
    P = T * k
    rbh, rbf = H // 64 * 36, F // 64 * 36
    uniq = statistics.mean(D["uniq"])
    if decode:
        return [(moe.MOE_KERNEL_GU_DECODE, "gu_decode_kernel",
                 uniq * 2 * F * rbh + T * H * 2 + P * F * 4, "GB/s", HBM_PEAK_GBS),
                (moe.MOE_KERNEL_DN_DECODE, "dn_decode_kernel",
                 uniq * H * rbf + P * F * 4 + P * H * 4, "GB/s", HBM_PEAK_GBS)]
    return [(moe.MOE_KERNEL_GU_PREFILL, "gemm_kernel<false>", 4.0 * P * H * F, "TFLOP/s",
             F16_PEAK_TFLOPS),
            (moe.MOE_KERNEL_DN_PREFILL, "gemm_kernel<true>", 2.0 * P * H * F, "TFLOP/s",
             F16_PEAK_TFLOPS)]


def hbm_note(D, warm):
    E = D["E"]
    rbh, rbf = D["H"] // 64 * 36, D["F"] // 64 * 36
    per_expert = 2 * D["F"] * rbh + D["H"] * rbf
    cycled = min(E, sum(D["uniq"])) * per_expert * D["copies"]
    if warm:
        return "warm (one routing reused)"
    if cycled < 256e6:
        return (f"cache-resident: {cycled / 1e6:.1f} MB of weights in rotation, under the "
                "256 MB Infinity Cache")
    if len(D["ids"]) > 1 or D["copies"] > 1:
        return (f"cold ({len(D['ids'])} routings over disjoint expert windows x "
                f"{D['copies']} bank copies, {cycled / 1e6:.0f} MB of weights in rotation)")
    return f"cold ({cycled / 1e6:.0f} MB of weights per step, over 2 x the Infinity Cache)"


def measure(D, path_flag, K, W, q, torch, moe, kernels=True, two_calls=True):
    """Times one workload: per-layer GPU times over K steps of the one-call layer
    (moe_layer_nvfp4), the path's two big kernels, and for comparison the layer as two calls
    (moe_route_bucket + moe_ffn_nvfp4)."""
    T = D["T"]
    per2 = None
    if two_calls:
        two = Layer(D, path_flag, torch, moe, fused=False)
        for i in range(W):
            two.step(i)
        torch.cuda.synchronize()
        per2, span2, _ = time_steps(q, two.step, K, W)
        del two
    lay = Layer(D, path_flag, torch, moe)
    for i in range(W):
        lay.step(i)
    torch.cuda.synchronize()
    per, span, qinfo = time_steps(q, lay.step, K, W)
    H, F, k = D["H"], D["F"], D["k"]
    decode = path_flag == moe.MOE_PATH_DECODE or (
        path_flag == moe.MOE_PATH_AUTO and moe.moe_auto_path(T, k, D["E"], H, F) == moe.MOE_PATH_DECODE)
    rbh, rbf = H // 64 * 36, F // 64 * 36
    per_expert = 2 * F * rbh + H * rbf
    uniq = statistics.mean(D["uniq"])
    med = statistics.median(per)
    s = span * 1e-3
    res = {
        # mean: K back-to-back layers between two events; the rest: an event between every two
        "layer_us": {"mean": span * 1e3, "per_step_median": med * 1e3,
                     "per_step_min": min(per) * 1e3,
                     "per_step_spread": (max(per) - min(per)) / med if med > 0 else None},
        "ms_per_step": span, "decode": decode, "queue": qinfo,
        "two_call_layer_us": None if per2 is None else {
            "mean": span2 * 1e3, "per_step_median": statistics.median(per2) * 1e3},
        "unique_expert_bytes": uniq * per_expert,
        "unique_gbs": uniq * per_expert / s / 1e9,
        "hbm_frac_unique": uniq * per_expert / s / 1e9 / HBM_PEAK_GBS,
        "useful_tflops": 6.0 * T * k * H * F / s / 1e12,
        "mfma_frac_useful": 6.0 * T * k * H * F / s / 1e12 / F16_PEAK_TFLOPS,
        "kernels": {},
    }
    if kernels:
        for kid, kname, amount, unit, peak in kernel_table(D, decode):
            avg_ms, n = kernel_avg_ms(q, moe, kid, lay.step, K, W + K)
            ach = amount / (avg_ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
            res["kernels"][kname] = {"avg_launch_us": avg_ms * 1e3, "launches": n,
                                     "per_launch": amount, "achieved": ach, "unit": unit,
                                     "peak": peak, "frac": ach / peak}
    del lay
    return res


# ----------------------------------------------------------------------------------- main

def describe(D):
    E, H, F, k, T = D["E"], D["H"], D["F"], D["k"], D["T"]
    return {"verify_chunk": f"verify chunk: E={E} H={H} F={F} top-{k} T={T}, union U={D['U']}",
            "tiny_decode": f"tiny decode: E={E} H={H} F={F} top-{k} T={T}",
            "e256_plateau": f"rank-local E256 plateau: E={E} H={H} F={F} top-{k} T={T}",
            "skewed_prefill": f"skewed prefill: E={E} H={H} F={F} top-{k} T={T}",
            "full_prefill": f"full-width prefill: E={E} H={H} F={F} top-{k} T={T}",
            "shared_expert": f"shared expert (dense SwiGLU, every token): H={H} F={F} T={T}" +
                             (f", as {D['virtual']} caller-side virtual experts over its one "
                              f"weight copy" if D["virtual"] else ", E=1")}[D["name"]]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the routed layer here is one GPU's share; multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)

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
    q = Queue(torch)
    path = {"auto": moe.MOE_PATH_AUTO, "decode": moe.MOE_PATH_DECODE,
            "prefill": moe.MOE_PATH_PREFILL}[args.path]
    K, W = args.steps, args.warmup

    name = args.workload
    T = args.T or DEFAULT_T[name]
    t_wall = time.perf_counter()
    D = build_inputs(name, T, args.U if name == "verify_chunk" else None, args.warm, args.virtual,
                     torch, gen, moe, kpack=uses_gemm(gen, moe, name, T, path, args))
    res = measure(D, path, K, W, q, torch, moe, two_calls=not args.layer_only)
    decode = res["decode"]
    kname = "gu_decode_kernel" if decode else "gemm_kernel<false>"   # gate/up (+ SiLU)
    kr = res["kernels"][kname]
    if decode:
        value, unit = res["unique_gbs"], "GB/s"
        roof = {"bound": "hbm", "kernel": kname, "achieved": kr["achieved"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "bytes_per_launch": kr["per_launch"]}
    else:
        value, unit = res["useful_tflops"], "TFLOP/s"
        roof = {"bound": "mfma", "kernel": kname, "achieved": kr["achieved"],
                "peak": F16_PEAK_TFLOPS, "unit": "TFLOP/s", "flops_per_launch": kr["per_launch"]}
    roof.update(frac=kr["frac"], avg_launch_us=kr["avg_launch_us"], launches=kr["launches"])
    tr = measured_traffic(kname, D["name"], T, D["U"] if D["name"] == "verify_chunk" else None)
    roof["traffic"] = tr["bytes"] if tr else None
    if tr:
        roof["traffic_detail"] = tr

    desc, note = describe(D), hbm_note(D, args.warm)
    D_kpack = D["kpack"]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, D, unit)

    rows = []
    if args.rows == "all":
        host_banks = {name: D["host"]["banks"]}
        del D
        torch.cuda.empty_cache()
        for wl, Tr, Ur in ROWS:
            if wl not in host_banks:
                host_banks = {wl: make_banks_host(gen, wl)}   # one workload's banks at a time
            Dr = build_inputs(wl, Tr, Ur, args.warm, 0, torch, gen, moe, host_banks[wl],
                              kpack=uses_gemm(gen, moe, wl, Tr, moe.MOE_PATH_AUTO, args))
            r = measure(Dr, moe.MOE_PATH_AUTO, K, W, q, torch, moe, two_calls=not args.layer_only)
            r.update(workload=describe(Dr), name=wl, T=Tr, U=Dr["U"], E=Dr["E"], H=Dr["H"],
                     F=Dr["F"], top_k=Dr["k"], path="decode" if r["decode"] else "prefill",
                     hbm=hbm_note(Dr, args.warm),
                     gemm_weights="kpack" if Dr["kpack"] else "row-major")
            del r["decode"]
            rows.append(r)
            print(f"[row] {r['workload']}: {r['layer_us']['mean']:.1f} us per layer, "
                  f"{r['unique_gbs']:.0f} GB/s unique, {r['useful_tflops']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
            del Dr
            torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": desc, "T": T, "path": "decode" if decode else "prefill",
                   "hbm": note,
                   "gemm_weights": "kpack" if D_kpack else "row-major"},
        "layer": res["layer_us"],
        "two_call_layer_us": res["two_call_layer_us"],
        "unique_expert_bytes": res["unique_expert_bytes"],
        "hbm_frac_unique": res["hbm_frac_unique"],
        "useful_tflops": res["useful_tflops"],
        "queue": res["queue"],
        "roofline": roof,
        "kernels": res["kernels"],
        "cpu_baseline": cpu,
        "rows": rows,
        "wall_s": time.perf_counter() - t_wall,
    }
    print(json.dumps(out), flush=True)


def bench_router(args, torch, gen, moe):
    """The router step alone (moe_router_topk): fp32 logits [T, E] -> top-k ids and softmax
    weights. One step = one call over one logits batch; consecutive steps read different copies
    so that more than 2 x 256 MB cycle through (the logits come from HBM, not the Infinity Cache,
    where a batch is large enough for that to matter)."""
    import numpy as np
    import oracle

    q = Queue(torch)
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
    per, qinfo = time_steps(q, step, K, args.warmup)
    ms_per_step = sum(per) / K
    k_ms, n_k = kernel_avg_ms(q, moe, moe.MOE_KERNEL_ROUTER, step, K, args.warmup + K)
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
               "seconds_per_batch": sec, "reps": reps, **host_info()}
    out = {
        "metric": "router step µs + GB/s of logits read and ids/weights written",
        "value": nbytes / s / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"router top-{k}: E={E} T={T}, N(0,1) fp32 logits", "E": E,
                   "top_k": k, "T": T, "hbm": f"{copies} logits copies in rotation"},
        "step_us": ms_per_step * 1e3, "queue": qinfo,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def host_info():
    """CPU model and core counts of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_available": avail}


def cpu_baseline(args, D, unit):
    """The fp64 oracle (union form: each active expert decoded once, the experts shared out over
    the threads) timed on the host cores on a bounded sample of the same workload, scaled to the
    metric's unit; and once on one thread on the first token, for comparison. Threads: every
    core this process may run on, up to OMP_NUM_THREADS when that is set (the host's CPU share)."""
    import numpy as np

    import oracle
    hi = host_info()
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(hi["cpus_available"], cap) if cap > 0 else hi["cpus_available"]
    name = D["name"]
    E, H, F, k, T = D.get("oracle_E", D["E"]), D["H"], D["F"], D["k"], D["T"]
    ids = D.get("oracle_ids", D["variants"][0])
    per_expert = 2 * F * (H // 64 * 36) + H * (F // 64 * 36)
    case = dict(E=E, H=H, F=F, k=k, T=T, ids=ids, w=D["host"]["w"], x=D["host"]["x"],
                **D["host"]["banks"])
    if T * k <= 1280:
        tok = None
        sample = f"whole layer (all {T} tokens, {T * k} routed slots)"
    else:
        tok = np.arange(8)
        sample = f"8 of the layer's {T} tokens ({8 * k} routed slots)"

    def rate(sec_, tokens):
        sel = ids if tokens is None else ids[tokens]
        if unit == "GB/s":
            return len(np.unique(sel)) * per_expert / sec_ / 1e9
        return 6.0 * sel.size * H * F / sec_ / 1e12

    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.ffn_union(case, threads=threads, tokens=tok)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or el * (reps + 1) / reps > 30.0:
            break
    sec = el / reps
    t1 = time.perf_counter()
    one = np.arange(1)
    oracle.ffn_union(case, threads=1, tokens=one)
    sec1 = time.perf_counter() - t1
    single = {"value": rate(sec1, one), "cores": 1,
              "sample": f"the first token ({k} routed slots), once", "seconds_per_sample": sec1}
    return {"value": rate(sec, tok), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": sample + ", union form", "seconds_per_sample": sec, "reps": reps,
            "single_thread": single, **hi}


if __name__ == "__main__":
    main()
