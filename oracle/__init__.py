"""TEST INFRASTRUCTURE ONLY: ctypes wrapper over the fp64 C oracle (moe_oracle.c).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
The GPU library never does, and the oracle never touches the GPU library.

Functions follow the definitions cited in moe_oracle.c. Every function here is pinned by a
CPU test against something other than itself (see tests/test_oracle_pins.py):
  e2m1 / ue4m3 / nvfp4 decode  - the OCP element tables and torch's float8_e4m3fn decoding;
  route_bucket                 - a stable sort of the pair list (Python's sorted) and invariants;
  router_topk                  - numpy's stable sort and scipy's softmax, closed forms, ties;
  ffn_per_slot / ffn_union     - numpy float64 matmuls on independently decoded weights (with
                                 and without second-level scales), closed-form special cases,
                                 invariances.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        lib.orc_e2m1.restype = ctypes.c_double
        lib.orc_e2m1.argtypes = [ctypes.c_int]
        lib.orc_ue4m3.restype = ctypes.c_double
        lib.orc_ue4m3.argtypes = [ctypes.c_int]
        lib.orc_bf16.restype = ctypes.c_double
        lib.orc_bf16.argtypes = [ctypes.c_uint16]
        lib.orc_nvfp4_weight.restype = ctypes.c_double
        lib.orc_nvfp4_weight.argtypes = [_u8p, ctypes.c_int64]
        lib.orc_dequant_rows.restype = None
        lib.orc_dequant_rows.argtypes = [_u8p, ctypes.c_int64, ctypes.c_int64, _f64p]
        lib.orc_route_bucket.restype = ctypes.c_int
        lib.orc_route_bucket.argtypes = [_i32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _i32p, _i32p, _i32p, _i32p]
        lib.orc_ffn_per_slot_s2.restype = ctypes.c_int
        lib.orc_ffn_per_slot_s2.argtypes = [
            _u16p, _f32p, _i32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, _u8p, ctypes.c_int64, _u8p, ctypes.c_int64, _u8p,
            ctypes.c_int64, _f32p, _f32p, _f32p, _i64p, ctypes.c_int64, _f64p, ctypes.c_int32]
        lib.orc_router_topk.restype = ctypes.c_int
        lib.orc_router_topk.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        _i32p, _f64p]
        lib.orc_set_h_round.restype = None
        lib.orc_set_h_round.argtypes = [ctypes.c_int32]
        lib.orc_ffn_union_sel_s2.restype = ctypes.c_int
        lib.orc_ffn_union_sel_s2.argtypes = [
            _u16p, _f32p, _i32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, _u8p, ctypes.c_int64, _u8p, ctypes.c_int64, _u8p,
            ctypes.c_int64, _f32p, _f32p, _f32p, _i64p, ctypes.c_int64, _f64p, _f64p,
            ctypes.c_int32]
        _lib = lib
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def e2m1(code: int) -> float:
    return _load().orc_e2m1(int(code))


def ue4m3(byte: int) -> float:
    return _load().orc_ue4m3(int(byte))


def bf16(bits: int) -> float:
    return _load().orc_bf16(int(bits))


def dequant_rows(rows: np.ndarray, in_f: int) -> np.ndarray:
    """Decode uint8 NVFP4 rows [n, row_bytes] into float64 [n, in_f]."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.size // (in_f // 64 * 36)
    out = np.empty((n, in_f), dtype=np.float64)
    _load().orc_dequant_rows(_p(rows, _u8p), n, in_f, _p(out, _f64p))
    return out


def route_bucket(ids: np.ndarray, E: int, expert_base: int = 0):
    """Returns (offsets[E+1], pair_ids[offsets[E]], active[n_active], n_active, n_nonlocal)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    P = T * k
    offsets = np.zeros(E + 1, dtype=np.int32)
    pair_ids = np.zeros(max(P, 1), dtype=np.int32)
    active = np.zeros(E, dtype=np.int32)
    counts = np.zeros(2, dtype=np.int32)
    rc = _load().orc_route_bucket(_p(ids, _i32p), T, k, E, expert_base, _p(offsets, _i32p),
                                  _p(pair_ids, _i32p), _p(active, _i32p), _p(counts, _i32p))
    if rc:
        raise ValueError("orc_route_bucket rejected its arguments")
    n_local = int(offsets[E])
    return offsets, pair_ids[:n_local].copy(), active[:counts[0]].copy(), int(counts[0]), int(counts[1])


def router_topk(logits: np.ndarray, k: int):
    """(ids int32 [T, k], w float64 [T, k]) from fp32 logits [T, E]: the k largest logits of each
    row in descending order (equal logits in ascending expert id), w the softmax over them."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    rc = _load().orc_router_topk(_p(logits, _f32p), T, E, k, _p(ids, _i32p), _p(w, _f64p))
    if rc:
        raise ValueError("orc_router_topk rejected its arguments")
    return ids, w


def bank_views(case: dict):
    """(gate, gate_stride, up, up_stride, down, down_stride) host views for a workload dict
    from gen.inputs: fused gate_up banks give gate = rows [0,F), up = rows [F,2F) of each expert."""
    F, H = case["F"], case["H"]
    rbh = H // 64 * 36
    if "gate_up" in case:
        gu = np.ascontiguousarray(case["gate_up"])
        stride = 2 * F * rbh
        flat = gu.reshape(-1)
        gate = flat
        up = flat[F * rbh:]
        return gate, stride, up, stride, np.ascontiguousarray(case["down"]).reshape(-1), H * (F // 64 * 36)
    gate = np.ascontiguousarray(case["gate"]).reshape(-1)
    up = np.ascontiguousarray(case["up"]).reshape(-1)
    return gate, F * rbh, up, F * rbh, np.ascontiguousarray(case["down"]).reshape(-1), H * (F // 64 * 36)


def _s2(case: dict):
    """The case's second-level scales (float32 [E] per bank under gate_s2 / up_s2 / down_s2),
    each as a ctypes pointer or None, plus the arrays to keep alive."""
    keep, ptrs = [], []
    for key in ("gate_s2", "up_s2", "down_s2"):
        a = case.get(key)
        if a is None:
            ptrs.append(None)
        else:
            a = np.ascontiguousarray(a, dtype=np.float32)
            if a.size != case["E"]:
                raise ValueError(f"{key} needs one scale per expert")
            keep.append(a)
            ptrs.append(_p(a, _f32p))
    return ptrs, keep


H_ROUND = {"none": 0, "bf16": 1, "hi_lo": 2}


class _HRound:
    """Sets the oracle's diagnostic rounding of h for one call and restores the canonical mode
    (h unrounded) afterwards, whatever happens."""

    def __init__(self, lib, mode: str):
        self.lib, self.mode = lib, H_ROUND[mode]

    def __enter__(self):
        self.lib.orc_set_h_round(self.mode)

    def __exit__(self, *exc):
        self.lib.orc_set_h_round(0)


def ffn_per_slot(case: dict, tokens=None, threads: int = 0, expert_base: int | None = None,
                 h_round: str = "none"):
    """fp64 y[len(tokens), H] (all tokens when tokens is None), per-slot form. h_round is the
    diagnostic rounding of the intermediate h: "none" (canonical), "bf16" or "hi_lo"."""
    lib = _load()
    x = np.ascontiguousarray(case["x"], dtype=np.uint16)
    w = np.ascontiguousarray(case["w"], dtype=np.float32)
    ids = np.ascontiguousarray(case["ids"], dtype=np.int32)
    T, k = ids.shape
    E, H, F = case["E"], case["H"], case["F"]
    eb = case.get("expert_base", 0) if expert_base is None else expert_base
    gate, gs, up, us, down, ds = bank_views(case)
    if tokens is None:
        tok_p, n = None, T
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int64)
        tok_p, n = _p(tok, _i64p), tok.size
    y = np.zeros((n, H), dtype=np.float64)
    s2, _keep = _s2(case)
    with _HRound(lib, h_round):
        rc = lib.orc_ffn_per_slot_s2(_p(x, _u16p), _p(w, _f32p), _p(ids, _i32p), T, k, E, eb, H,
                                     F, _p(gate, _u8p), gs, _p(up, _u8p), us, _p(down, _u8p), ds,
                                     *s2, tok_p, n, _p(y, _f64p), threads)
    if rc:
        raise ValueError("orc_ffn_per_slot rejected its arguments")
    return y


def ffn_union(case: dict, threads: int = 0, expert_base: int | None = None, want_h: bool = False,
              h_round: str = "none", tokens=None):
    """fp64 y[T, H], union form (optionally also h[T*k, F] for computed local pairs, NaN
    elsewhere). tokens: compute only these tokens' pairs and return their rows y[len(tokens), H]
    (each bit for bit as in the full layer). h_round as for ffn_per_slot."""
    lib = _load()
    x = np.ascontiguousarray(case["x"], dtype=np.uint16)
    w = np.ascontiguousarray(case["w"], dtype=np.float32)
    ids = np.ascontiguousarray(case["ids"], dtype=np.int32)
    T, k = ids.shape
    E, H, F = case["E"], case["H"], case["F"]
    eb = case.get("expert_base", 0) if expert_base is None else expert_base
    gate, gs, up, us, down, ds = bank_views(case)
    if tokens is None:
        tok_p, n = None, T
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int64)
        tok_p, n = _p(tok, _i64p), tok.size
    y = np.zeros((n, H), dtype=np.float64)
    h = np.full((T * k, F), np.nan) if want_h else None
    s2, _keep = _s2(case)
    with _HRound(lib, h_round):
        rc = lib.orc_ffn_union_sel_s2(_p(x, _u16p), _p(w, _f32p), _p(ids, _i32p), T, k, E, eb, H,
                                      F, _p(gate, _u8p), gs, _p(up, _u8p), us, _p(down, _u8p),
                                      ds, *s2, tok_p, n, _p(y, _f64p),
                                      _p(h, _f64p) if want_h else None, threads)
    if rc:
        raise ValueError("orc_ffn_union rejected its arguments")
    return (y, h) if want_h else y
