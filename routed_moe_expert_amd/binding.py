"""ctypes binding of libmoe_nvfp4.so: same entry points as include/moe_nvfp4.h.

Argument marshalling only: tensors become device pointers, the stream becomes a hipStream_t.
Every step of the layer runs in the library's HIP kernels. Importing this module fails loudly
when the library has not been built.
"""
from __future__ import annotations

import ctypes
import importlib.util
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_nvfp4.so")

MOE_OK, MOE_EINVAL, MOE_EWS, MOE_ESHAPE, MOE_ELAUNCH = 0, 1, 2, 3, 4
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL = 0, 1, 2
MOE_AUTO_PAIRS_PER_EXPERT = 16
MOE_KPACK_ROWS = 256
(MOE_KERNEL_NONE, MOE_KERNEL_BUCKET, MOE_KERNEL_GU_DECODE, MOE_KERNEL_DN_DECODE, MOE_KERNEL_COMBINE,
 MOE_KERNEL_SCHEDULE, MOE_KERNEL_GU_PREFILL, MOE_KERNEL_DN_PREFILL, MOE_KERNEL_ROUTER) = range(9)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {moe_status_str(status)} ({status})")
        self.status = status


class moe_bank(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("expert_stride", ctypes.c_int64),
                ("scale2", ctypes.c_void_p), ("experts", ctypes.c_void_p),
                ("kpack", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python routed_moe_expert_amd/build.py` (hipcc, gfx950)")
    # One HIP runtime per process: PyTorch ships its own libamdhip64 (same soname, loaded under
    # another file name). Loaded after ours, it would be a second runtime that knows nothing of
    # our kernels' module or of the other's allocations; loaded first, ours binds to it.
    if importlib.util.find_spec("torch") is not None:
        import torch  # noqa: F401
    l = ctypes.CDLL(LIB_PATH)
    i32, sz, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    l.moe_route_bucket_ws.restype = sz
    l.moe_route_bucket_ws.argtypes = [i32, i32, i32]
    l.moe_route_bucket.restype = ctypes.c_int
    l.moe_route_bucket.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    l.moe_ffn_nvfp4_ws.restype = sz
    l.moe_ffn_nvfp4_ws.argtypes = [i32, i32, i32, i32, i32]
    l.moe_auto_path.restype = i32
    l.moe_auto_path.argtypes = [i32, i32, i32, i32, i32]
    l.moe_ffn_nvfp4.restype = ctypes.c_int
    l.moe_ffn_nvfp4.argtypes = [vp, vp, vp, vp, vp, vp, moe_bank, moe_bank, moe_bank,
                                i32, i32, i32, i32, i32, vp, i32, vp, sz, vp]
    l.moe_layer_nvfp4_ws.restype = sz
    l.moe_layer_nvfp4_ws.argtypes = [i32, i32, i32, i32, i32]
    l.moe_layer_nvfp4.restype = ctypes.c_int
    l.moe_layer_nvfp4.argtypes = [vp, i32, vp, vp, moe_bank, moe_bank, moe_bank, i32, i32, i32,
                                  i32, i32, vp, i32, vp, sz, vp]
    l.moe_ffn_nvfp4_static.restype = ctypes.c_int
    l.moe_ffn_nvfp4_static.argtypes = [vp, vp, vp, vp, vp, vp, moe_bank, moe_bank, moe_bank,
                                       i32, i32, i32, i32, i32, vp, i32, vp]
    l.moe_kpack_bytes.restype = sz
    l.moe_kpack_bytes.argtypes = [i32, i32, i32]
    l.moe_kpack.restype = ctypes.c_int
    l.moe_kpack.argtypes = [moe_bank, i32, i32, i32, vp, vp]
    l.moe_router_topk.restype = ctypes.c_int
    l.moe_router_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    l.moe_profile_kernel.restype = ctypes.c_int
    l.moe_profile_kernel.argtypes = [i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32]
    l.moe_profile_count.restype = i32
    l.moe_profile_count.argtypes = []
    l.moe_status_str.restype = ctypes.c_char_p
    l.moe_status_str.argtypes = [ctypes.c_int]
    return l


lib = _load()


def _ptr(t) -> int:
    """Device address of a tensor (or an int address / None)."""
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int, raise_on_error: bool) -> int:
    if status != MOE_OK and raise_on_error:
        raise MoeError(fn, status)
    return status


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(int(status)).decode()


def moe_route_bucket_ws(T: int, k: int, E: int) -> int:
    return int(lib.moe_route_bucket_ws(T, k, E))


def moe_ffn_nvfp4_ws(T: int, k: int, E: int, H: int, F: int) -> int:
    return int(lib.moe_ffn_nvfp4_ws(T, k, E, H, F))


def moe_auto_path(T: int, k: int, E: int, H: int, F: int) -> int:
    """The path MOE_PATH_AUTO takes for these sizes (host only); raises on refused sizes."""
    p = int(lib.moe_auto_path(T, k, E, H, F))
    if p < 0:
        raise MoeError("moe_auto_path", -p)
    return p


def moe_route_bucket(topk_ids, T: int, k: int, E: int, expert_base: int, offsets, pair_ids,
                     active, counts, ws=None, ws_bytes: int = 0, stream=None,
                     raise_on_error: bool = True) -> int:
    st = lib.moe_route_bucket(_ptr(topk_ids), T, k, E, expert_base, _ptr(offsets), _ptr(pair_ids),
                              _ptr(active), _ptr(counts), _ptr(ws), ws_bytes, _stream(stream))
    return _check("moe_route_bucket", st, raise_on_error)


def bank(base, expert_stride: int, byte_offset: int = 0, scale2=None, experts=None,
         kpack=None) -> moe_bank:
    """A moe_bank for a device tensor (or address) plus an optional byte offset, and optionally
    the bank's per-expert fp32 second-level scales (a device tensor of E floats), a per-expert
    pointer table (a device int64 tensor of E addresses; base and expert_stride are then unused)
    and a K-step-packed copy of the same weights for the GEMM path (a device uint8 tensor that
    moe_kpack wrote).

    The bank holds raw addresses, so it also keeps a reference to every tensor it was given
    (`_keep`): their memory cannot be freed and reused while the bank object is alive. Addresses
    passed as ints are the caller's to keep valid."""
    b = moe_bank(_ptr(base) + byte_offset if base is not None else None, int(expert_stride),
                 _ptr(scale2) or None, _ptr(experts) or None, _ptr(kpack) or None)
    b._keep = tuple(t for t in (base, scale2, experts, kpack)
                    if t is not None and not isinstance(t, int))
    return b


def moe_kpack_bytes(E: int, out_f: int, in_f: int) -> int:
    return int(lib.moe_kpack_bytes(E, out_f, in_f))


def moe_kpack(src: moe_bank, E: int, out_f: int, in_f: int, dst, stream=None,
              raise_on_error: bool = True) -> int:
    st = lib.moe_kpack(src, E, out_f, in_f, _ptr(dst), _stream(stream))
    return _check("moe_kpack", st, raise_on_error)


def with_kpack(src: moe_bank, E: int, out_f: int, in_f: int, stream=None) -> moe_bank:
    """A copy of bank src that also carries its K-step-packed copy (allocated here as a device
    uint8 tensor and written by moe_kpack on the stream)."""
    import torch
    dst = torch.empty(moe_kpack_bytes(E, out_f, in_f), dtype=torch.uint8, device="cuda")
    moe_kpack(src, E, out_f, in_f, dst, stream)
    b = moe_bank(src.base, src.expert_stride, src.scale2, src.experts, dst.data_ptr())
    b._keep = getattr(src, "_keep", ()) + (dst,)
    return b


def moe_ffn_nvfp4(x, topk_w, offsets, pair_ids, active, counts, gate: moe_bank, up: moe_bank,
                  down: moe_bank, T: int, k: int, E: int, H: int, F: int, y, path: int = MOE_PATH_AUTO,
                  ws=None, ws_bytes: int = 0, stream=None, raise_on_error: bool = True) -> int:
    st = lib.moe_ffn_nvfp4(_ptr(x), _ptr(topk_w), _ptr(offsets), _ptr(pair_ids), _ptr(active),
                           _ptr(counts), gate, up, down, T, k, E, H, F, _ptr(y), path, _ptr(ws),
                           ws_bytes, _stream(stream))
    return _check("moe_ffn_nvfp4", st, raise_on_error)


def moe_layer_nvfp4_ws(T: int, k: int, E: int, H: int, F: int) -> int:
    return int(lib.moe_layer_nvfp4_ws(T, k, E, H, F))


def moe_layer_nvfp4(topk_ids, expert_base: int, x, topk_w, gate: moe_bank, up: moe_bank,
                    down: moe_bank, T: int, k: int, E: int, H: int, F: int, y,
                    path: int = MOE_PATH_AUTO, ws=None, ws_bytes: int = 0, stream=None,
                    raise_on_error: bool = True) -> int:
    st = lib.moe_layer_nvfp4(_ptr(topk_ids), expert_base, _ptr(x), _ptr(topk_w), gate, up, down,
                             T, k, E, H, F, _ptr(y), path, _ptr(ws), ws_bytes, _stream(stream))
    return _check("moe_layer_nvfp4", st, raise_on_error)


MOE_STATIC_WS_BYTES = 128 << 20


def moe_ffn_nvfp4_static(x, topk_w, offsets, pair_ids, active, counts, gate: moe_bank,
                         up: moe_bank, down: moe_bank, T: int, k: int, E: int, H: int, F: int, y,
                         path: int = MOE_PATH_AUTO, stream=None, raise_on_error: bool = True) -> int:
    st = lib.moe_ffn_nvfp4_static(_ptr(x), _ptr(topk_w), _ptr(offsets), _ptr(pair_ids),
                                  _ptr(active), _ptr(counts), gate, up, down, T, k, E, H, F,
                                  _ptr(y), path, _stream(stream))
    return _check("moe_ffn_nvfp4_static", st, raise_on_error)


def moe_router_topk(logits, T: int, E: int, k: int, topk_ids, topk_w, stream=None,
                    raise_on_error: bool = True) -> int:
    st = lib.moe_router_topk(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _stream(stream))
    return _check("moe_router_topk", st, raise_on_error)


def moe_profile_kernel(kernel_id: int, start_events, stop_events) -> int:
    """start_events / stop_events: sequences of raw hipEvent_t handles (ints)."""
    n = len(start_events)
    arr = ctypes.c_void_p * max(n, 1)
    _profile_keep[:] = [arr(*start_events), arr(*stop_events)]
    st = lib.moe_profile_kernel(kernel_id, _profile_keep[0], _profile_keep[1], n)
    return _check("moe_profile_kernel", st, True)


def moe_profile_count() -> int:
    return int(lib.moe_profile_count())


_profile_keep = []
