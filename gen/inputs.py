"""Seeded synthetic inputs for the routed NVFP4 MoE FFN workloads.

Every buffer comes from its own counter-based Philox stream, keyed by (seed, stream id), so a
buffer can be regenerated alone. Nothing here evaluates the layer: the generator only lays
down bytes and numbers with the shapes and value distributions of the workloads that the
memra-engine probes and the Rocket E256 post measure (weights, activations, routing, router
weights).

NVFP4 block layout written here (64 weights in 36 bytes: four UE4M3 sub-scales, then 32 code
bytes; moe_sel_census.rs, its block constants): bytes 0..3 of a block are the scale bytes, bytes 4..35 the
code bytes. Codes are uniform random bytes, so every E2M1 nibble is uniform over its 16 values.
"""
from __future__ import annotations

import numpy as np

NVFP4_BLOCK_WEIGHTS = 64
NVFP4_BLOCK_BYTES = 36
NVFP4_SCALES_PER_BLOCK = 4

# stream ids: one per buffer kind, so adding a buffer never shifts another's values
S_GATE, S_UP, S_DOWN, S_GATEUP, S_X, S_ROUTE, S_LOGITS, S_PERM = 1, 2, 3, 4, 5, 6, 7, 8
S_RLOGITS = 9
S_S2 = 10
S_SKEW = 11


def rng_for(seed: int, stream: int, sub: int = 0) -> np.random.Generator:
    """Counter-based Philox stream keyed by (seed, stream, sub)."""
    key = np.array([(int(seed) << 20) ^ (int(sub) & 0xFFFFF), int(stream)], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def row_bytes(in_f: int) -> int:
    """Bytes of one NVFP4 row of in_f weights (in_f must be a multiple of 64)."""
    if in_f % NVFP4_BLOCK_WEIGHTS:
        raise ValueError("in_f must be a multiple of 64")
    return in_f // NVFP4_BLOCK_WEIGHTS * NVFP4_BLOCK_BYTES


def nvfp4_bank(seed: int, stream: int, n_expert: int, out_f: int, in_f: int,
               scales: str = "pow2") -> np.ndarray:
    """Expert-major NVFP4 bank, uint8 [n_expert, out_f, row_bytes(in_f)].

    scales:
      "pow2" - every scale byte is 2^e with e uniform in {-6..2} (UE4M3 bytes 0x08..0x48,
               mantissa 0), the distribution of the tiny-decode workload;
      "all"  - scale bytes uniform over all 127 finite UE4M3 codes 0x00..0x7E (subnormals,
               mantissas and zero included);
      "ones" - every scale 1.0 (byte 0x38).
    """
    rb = row_bytes(in_f)
    nblk = n_expert * out_f * (in_f // NVFP4_BLOCK_WEIGHTS)
    rng = rng_for(seed, stream)
    bank = np.frombuffer(rng.bytes(nblk * NVFP4_BLOCK_BYTES), dtype=np.uint8).copy()
    blocks = bank.reshape(nblk, NVFP4_BLOCK_BYTES)
    srng = rng_for(seed, stream, 1)
    if scales == "pow2":
        e_field = srng.integers(1, 10, size=(nblk, NVFP4_SCALES_PER_BLOCK), dtype=np.uint8)
        blocks[:, :NVFP4_SCALES_PER_BLOCK] = e_field << 3
    elif scales == "all":
        blocks[:, :NVFP4_SCALES_PER_BLOCK] = srng.integers(
            0, 127, size=(nblk, NVFP4_SCALES_PER_BLOCK), dtype=np.uint8)
    elif scales == "ones":
        blocks[:, :NVFP4_SCALES_PER_BLOCK] = 0x38
    else:
        raise ValueError(scales)
    return bank.reshape(n_expert, out_f, rb)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_normal(seed: int, shape, stream: int = S_X) -> np.ndarray:
    """bf16 bit patterns of N(0,1) samples (drawn in float32, rounded to nearest even)."""
    z = rng_for(seed, stream).standard_normal(size=shape, dtype=np.float32)
    return f32_to_bf16_bits(z)


def router_weights(seed: int, T: int, k: int) -> np.ndarray:
    """Softmax over each token's k N(0,1) logits, in float64, rounded once to float32."""
    z = rng_for(seed, S_LOGITS).standard_normal(size=(T, k))
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    return p.astype(np.float32)


def router_logits(seed: int, T: int, E: int, ties: bool = False) -> np.ndarray:
    """float32 [T, E] N(0,1) router logits. ties=True rounds them to multiples of 1/4, so that
    equal logits (and ties at the k-th place) are common."""
    z = rng_for(seed, S_RLOGITS).standard_normal(size=(T, E), dtype=np.float32)
    if ties:
        z = np.round(z * 4.0).astype(np.float32) / np.float32(4.0)
    return np.ascontiguousarray(z, dtype=np.float32)


def route_distinct(seed: int, T: int, k: int, E: int) -> np.ndarray:
    """k distinct experts per token, drawn uniformly without replacement (int32 [T,k])."""
    rng = rng_for(seed, S_ROUTE)
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False)
    return out


def route_union(seed: int, T: int, k: int, E: int, U: int) -> np.ndarray:
    """Fixed slot count, swept union: slot (t,j) -> pi_U[(t*k+j) mod U], pi_U a seeded
    U-subset of the E experts. With U >= k no token names an expert twice."""
    if not (k <= U <= E):
        raise ValueError("need k <= U <= E")
    pi = rng_for(seed, S_PERM, U).choice(E, size=U, replace=False)
    p = np.arange(T * k)
    return pi[p % U].astype(np.int32).reshape(T, k)


def route_union_rotated(seed: int, T: int, k: int, E: int, U: int, variant: int) -> np.ndarray:
    """Like route_union, with the U-subset taken as the variant-th window of U experts of one
    seeded permutation (windows wrap around E), so consecutive variants touch disjoint experts.
    Benchmarks rotate variants so that an expert's bytes are not still cached from a recent call."""
    if not (k <= U <= E):
        raise ValueError("need k <= U <= E")
    perm = rng_for(seed, S_PERM, 1 << 19).permutation(E)
    pi = perm[(variant * U + np.arange(U)) % E]
    p = np.arange(T * k)
    return pi[p % U].astype(np.int32).reshape(T, k)


def route_cyclic(seed: int, T: int, k: int, E: int) -> np.ndarray:
    """Uniform routing that activates every expert as soon as T*k >= E:
    slot (t,j) -> pi[(t*k+j) mod E], pi a seeded permutation of the E experts."""
    pi = rng_for(seed, S_PERM).permutation(E)
    p = np.arange(T * k)
    return pi[p % E].astype(np.int32).reshape(T, k)


def route_skewed(T: int, k: int, E: int, seed: int = 0) -> np.ndarray:
    """Skewed routing of the moe_sk_repro probe's prefill workload: pair p = t*k + j goes to
    expert min(floor(u_p^1.35 * E), E - 1), u_p uniform in [0, 1). u_p is the p-th double of a
    Philox stream (53 bits of its p-th 64-bit output), i.e. a counter-based 64-bit hash of p:
    a pure function of (seed, p), so a longer batch extends a shorter one."""
    u = rng_for(seed, S_SKEW).random(T * k)
    e = np.minimum(np.floor(np.power(u, 1.35) * E).astype(np.int64), E - 1)
    return e.astype(np.int32).reshape(T, k)


# --------------------------------------------------------------------------------------------
# Named workloads.  Each returns a dict of host arrays plus the shape parameters.
# --------------------------------------------------------------------------------------------

WORKLOADS = {
    # name: (E, H, F, k, fused gate_up bank?, scale distribution, seed)
    "tiny_decode": dict(E=64, H=2560, F=640, k=10, fused=True, seed=1),
    "verify_chunk": dict(E=512, H=2560, F=640, k=10, fused=True, seed=2),
    "e256_plateau": dict(E=256, H=2560, F=640, k=10, fused=True, seed=3),
    "skewed_prefill": dict(E=288, H=4096, F=640, k=8, fused=False, seed=4),
    "full_prefill": dict(E=288, H=4096, F=1280, k=8, fused=False, seed=5),
    # the shared expert (Rocket post: N320 beside the routed experts) as a one-expert layer
    "shared_expert": dict(E=1, H=2560, F=320, k=1, fused=False, seed=6),
}


def make_banks(E: int, H: int, F: int, fused: bool, seed: int, scales: str = "pow2"):
    """Weight banks. fused: gate_up [E, 2F, rb(H)] (rows [0,F) gate, [F,2F) up) plus down
    [E, H, rb(F)]; otherwise separate gate [E,F,rb(H)], up [E,F,rb(H)], down [E,H,rb(F)]."""
    banks = {}
    if fused:
        banks["gate_up"] = nvfp4_bank(seed, S_GATEUP, E, 2 * F, H, scales)
    else:
        banks["gate"] = nvfp4_bank(seed, S_GATE, E, F, H, scales)
        banks["up"] = nvfp4_bank(seed, S_UP, E, F, H, scales)
    banks["down"] = nvfp4_bank(seed, S_DOWN, E, H, F, scales)
    return banks


def make_routing(name: str, T: int, U: int | None = None, seed: int | None = None):
    w = WORKLOADS[name]
    s = w["seed"] if seed is None else seed
    E, k = w["E"], w["k"]
    if name == "tiny_decode":
        ids = route_distinct(s, T, k, E)
    elif name == "verify_chunk":
        ids = route_union(s, T, k, E, U if U is not None else T * k)
    elif name == "e256_plateau":
        ids = route_cyclic(s, T, k, E)
    elif name == "shared_expert":   # every token, one slot, weight 1
        return np.zeros((T, 1), dtype=np.int32), np.ones((T, 1), dtype=np.float32)
    else:
        ids = route_skewed(T, k, E)
    return ids, router_weights(s, T, k)


def make_workload(name: str, T: int, U: int | None = None, scales: str = "pow2",
                  seed: int | None = None, with_banks: bool = True):
    """Full synthetic input set for one named workload at T tokens."""
    w = WORKLOADS[name]
    s = w["seed"] if seed is None else seed
    ids, wts = make_routing(name, T, U, s)
    out = dict(name=name, E=w["E"], H=w["H"], F=w["F"], k=w["k"], T=T, fused=w["fused"],
               ids=ids, w=wts, x=bf16_normal(s, (T, w["H"])))
    if with_banks:
        out.update(make_banks(w["E"], w["H"], w["F"], w["fused"], s, scales))
    return out


def make_random_case(seed: int, T: int, k: int, E: int, H: int, F: int,
                     scales: str = "all", nonlocal_frac: float = 0.0, expert_base: int = 0,
                     fused: bool = False):
    """Small random case for parity sweeps: i.i.d. uniform expert ids (duplicates within a
    token allowed), optionally with a fraction of ids outside [expert_base, expert_base+E)."""
    rng = rng_for(seed, S_ROUTE, 7)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int64) + expert_base
    if nonlocal_frac > 0:
        m = rng.random(size=(T, k)) < nonlocal_frac
        far = rng.integers(E, 2 * E + 3, size=(T, k)) + expert_base
        far = np.where(rng.random(size=(T, k)) < 0.5, far, expert_base - 1 - rng.integers(0, E, size=(T, k)))
        ids = np.where(m, far, ids)
    out = dict(E=E, H=H, F=F, k=k, T=T, fused=fused, expert_base=expert_base,
               ids=ids.astype(np.int32), w=router_weights(seed, T, k),
               x=bf16_normal(seed, (T, H)))
    out.update(make_banks(E, H, F, fused, seed, scales))
    return out


def make_shared_case(seed: int, T: int, H: int, F: int, scales: str = "pow2"):
    """The shared expert as a case of the routed layer: one expert (E = 1) that every token
    takes in its only slot (k = 1) with router weight 1, so the layer is the dense SwiGLU FFN
    y_t = Wd (silu(Wg x_t) * Wu x_t) over all T rows. Separate gate, up and down banks."""
    out = dict(E=1, H=H, F=F, k=1, T=T, fused=False, expert_base=0,
               ids=np.zeros((T, 1), dtype=np.int32), w=np.ones((T, 1), dtype=np.float32),
               x=bf16_normal(seed, (T, H)))
    out.update(make_banks(1, H, F, False, seed, scales))
    return out


def shared_virtual_routing(T: int, G: int):
    """The shared expert's tokens dealt round-robin to G virtual experts (token t -> t mod G), one
    slot each with router weight 1. With every virtual expert's bank rows pointing at the one
    expert's copy (a per-expert pointer table), the routed layer computes the same dense SwiGLU,
    with G times as many independent work items."""
    ids = (np.arange(T, dtype=np.int32) % G).reshape(T, 1)
    return ids, np.ones((T, 1), dtype=np.float32)


def split_ff(case: dict, F1: int):
    """Split a separate-bank case along ff at F1 (a multiple of 64), as a tensor-parallel shard
    of the FFN would hold it: rows [0, F1) and [F1, F) of gate and up, and of each down row the
    NVFP4 blocks of input features [0, F1) and [F1, F). Pure byte slicing: two cases whose
    outputs add up to the original's (the down projection is linear in h)."""
    F = case["F"]
    if F1 % NVFP4_BLOCK_WEIGHTS or not 0 < F1 < F:
        raise ValueError("F1 must be a multiple of 64 strictly inside (0, F)")
    b1 = row_bytes(F1)
    a = dict(case, F=F1, gate=np.ascontiguousarray(case["gate"][:, :F1]),
             up=np.ascontiguousarray(case["up"][:, :F1]),
             down=np.ascontiguousarray(case["down"][:, :, :b1]))
    b = dict(case, F=F - F1, gate=np.ascontiguousarray(case["gate"][:, F1:]),
             up=np.ascontiguousarray(case["up"][:, F1:]),
             down=np.ascontiguousarray(case["down"][:, :, b1:]))
    return a, b


def second_level_scales(seed: int, E: int, banks=("gate_s2", "up_s2", "down_s2")):
    """Per-expert fp32 second-level scales for each bank (ModelOpt's two-level NVFP4 keeps one
    such factor per weight tensor): log-uniform in [2^-4, 2^4], so none is a power of two."""
    rng = rng_for(seed, S_S2)
    return {b: np.exp2(rng.uniform(-4.0, 4.0, size=E)).astype(np.float32) for b in banks}
