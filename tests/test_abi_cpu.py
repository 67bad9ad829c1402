"""The C ABI without a GPU: the library loads, exports every declared entry point, sizes its
workspaces, and rejects bad arguments on the host before anything is enqueued."""
import os
import re

import numpy as np
import pytest

import routed_moe_expert_amd as moe
from routed_moe_expert_amd.binding import moe_bank

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000      # a 256-aligned non-null address; never dereferenced on these paths


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_\w+)\s*\(", src))
    return names


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"moe_route_bucket", "moe_ffn_nvfp4", "moe_route_bucket_ws", "moe_ffn_nvfp4_ws",
            "moe_router_topk", "moe_status_str"} <= names
    for n in names:
        assert hasattr(moe.lib, n), n


def test_status_strings():
    assert moe.moe_status_str(0) == "MOE_OK"
    assert moe.moe_status_str(moe.MOE_EWS) == "MOE_EWS"
    assert moe.moe_status_str(99) == "MOE_UNKNOWN"


def test_workspace_sizes():
    T, k, E, H, F = 6, 10, 512, 2560, 640
    P = T * k
    ws = moe.moe_ffn_nvfp4_ws(T, k, E, H, F)
    assert ws >= P * 4 + P * F * 4 + P * H * 4
    assert moe.moe_ffn_nvfp4_ws(4096, 8, 288, 4096, 1280) >= 32768 * 4096 * 4
    assert moe.moe_route_bucket_ws(T, k, E) >= 0
    assert moe.moe_ffn_nvfp4_ws(-1, 1, 1, 256, 64) == 0


def _bank(addr=FAKE, stride=4096):
    return moe_bank(addr, stride)


def _ffn(**over):
    a = dict(x=FAKE, topk_w=FAKE, offsets=FAKE, pair_ids=FAKE, active=FAKE, counts=FAKE,
             gate=_bank(), up=_bank(), down=_bank(), T=4, k=2, E=8, H=256, F=64, y=FAKE,
             path=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return moe.moe_ffn_nvfp4(a["x"], a["topk_w"], a["offsets"], a["pair_ids"], a["active"],
                             a["counts"], a["gate"], a["up"], a["down"], a["T"], a["k"], a["E"],
                             a["H"], a["F"], a["y"], a["path"], a["ws"], a["ws_bytes"], stream=0,
                             raise_on_error=False)


@pytest.mark.parametrize("over,status", [
    (dict(x=0), moe.MOE_EINVAL), (dict(y=0), moe.MOE_EINVAL), (dict(ws=0), moe.MOE_EINVAL),
    (dict(T=-1), moe.MOE_EINVAL), (dict(k=0), moe.MOE_EINVAL), (dict(E=0), moe.MOE_EINVAL),
    (dict(H=96), moe.MOE_EINVAL), (dict(H=0), moe.MOE_EINVAL), (dict(F=96), moe.MOE_EINVAL), (dict(path=7), moe.MOE_EINVAL), (dict(path=4), moe.MOE_EINVAL),
    (dict(gate=_bank(FAKE + 4)), moe.MOE_EINVAL), (dict(down=_bank(stride=100)), moe.MOE_EINVAL),
    (dict(up=_bank(0)), moe.MOE_EINVAL), (dict(x=FAKE + 2), moe.MOE_EINVAL),
    (dict(gate=moe_bank(0, 0, None, FAKE + 4)), moe.MOE_EINVAL),      # pointer table misaligned
    (dict(down=moe_bank(FAKE, 4096, FAKE + 2)), moe.MOE_EINVAL),      # scale2 misaligned
    (dict(ws=FAKE + 16), moe.MOE_EINVAL),
    (dict(gate=moe_bank(FAKE, 4096, None, None, FAKE + 8)), moe.MOE_EINVAL),  # kpack misaligned
    (dict(gate=moe_bank(FAKE, 4096, None, None, FAKE)), moe.MOE_EINVAL),  # gate packed, up not
    (dict(up=moe_bank(FAKE, 4096, None, None, FAKE)), moe.MOE_EINVAL),    # up packed, gate not
    (dict(E=4096), moe.MOE_ESHAPE), (dict(H=1 << 15), moe.MOE_ESHAPE),
    (dict(ws_bytes=16), moe.MOE_EWS),
    (dict(T=0), moe.MOE_OK), (dict(T=0, x=0, y=0), moe.MOE_OK),
])
def test_ffn_host_checks(over, status):
    assert _ffn(**over) == status


def _bucket(**over):
    a = dict(ids=FAKE, T=4, k=2, E=8, base=0, offsets=FAKE, pair_ids=FAKE, active=FAKE,
             counts=FAKE, ws=FAKE, ws_bytes=0)
    a.update(over)
    return moe.moe_route_bucket(a["ids"], a["T"], a["k"], a["E"], a["base"], a["offsets"],
                                a["pair_ids"], a["active"], a["counts"], a["ws"], a["ws_bytes"],
                                stream=0, raise_on_error=False)


@pytest.mark.parametrize("over,status", [
    (dict(ids=0), moe.MOE_EINVAL), (dict(offsets=0), moe.MOE_EINVAL),
    (dict(pair_ids=0), moe.MOE_EINVAL), (dict(counts=0), moe.MOE_EINVAL),
    (dict(T=-3), moe.MOE_EINVAL), (dict(k=0), moe.MOE_EINVAL), (dict(E=0), moe.MOE_EINVAL),
    (dict(E=5000), moe.MOE_ESHAPE), (dict(T=1 << 22, k=8), moe.MOE_ESHAPE),
])
def test_bucket_host_checks(over, status):
    assert _bucket(**over) == status


def test_errors_raise_by_default():
    with pytest.raises(moe.MoeError):
        moe.moe_route_bucket(0, 4, 2, 8, 0, 0, 0, 0, 0, stream=0)


def test_one_hip_runtime_whatever_the_import_order():
    """The package imported before torch must still leave a single HIP runtime mapped."""
    import subprocess
    import sys
    code = ("import routed_moe_expert_amd, torch\n"
            "paths = set()\n"
            "for line in open('/proc/self/maps'):\n"
            "    p = line.split()[-1]\n"
            "    if 'libamdhip64' in p: paths.add(p)\n"
            "print(len(paths))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_bucket_workspace_only_past_one_workgroup():
    """Up to 4096 pairs the bucketing runs in one workgroup's LDS; past that its chunked form
    keeps per-chunk histograms in the workspace, and a short workspace is refused on the host."""
    assert moe.moe_route_bucket_ws(512, 8, 288) == 0
    big = moe.moe_route_bucket_ws(4096, 8, 288)
    assert big > 0 and big % 256 == 0
    assert big >= 16 * 289 * 4          # at least 16 chunks of 289 bucket counts
    st = moe.lib.moe_route_bucket(FAKE, 4096, 8, 288, 0, FAKE, FAKE, FAKE, FAKE, FAKE, big - 256,
                                  None)
    assert st == moe.MOE_EWS
    st = moe.lib.moe_route_bucket(FAKE, 4096, 8, 288, 0, FAKE, FAKE, FAKE, FAKE, None, big, None)
    assert st == moe.MOE_EWS


def _router(**over):
    a = dict(logits=FAKE, T=4, E=64, k=8, ids=FAKE, w=FAKE)
    a.update(over)
    return moe.moe_router_topk(a["logits"], a["T"], a["E"], a["k"], a["ids"], a["w"], stream=0,
                               raise_on_error=False)


@pytest.mark.parametrize("over,status", [
    (dict(logits=0), moe.MOE_EINVAL), (dict(ids=0), moe.MOE_EINVAL), (dict(w=0), moe.MOE_EINVAL),
    (dict(T=-1), moe.MOE_EINVAL), (dict(E=0), moe.MOE_EINVAL), (dict(k=0), moe.MOE_EINVAL),
    (dict(k=65, E=64), moe.MOE_EINVAL), (dict(k=65, E=128), moe.MOE_ESHAPE),
    (dict(E=4096), moe.MOE_ESHAPE), (dict(T=1 << 22, k=8), moe.MOE_ESHAPE),
    (dict(T=0), moe.MOE_OK), (dict(T=0, logits=0, ids=0, w=0), moe.MOE_OK),
])
def test_router_host_checks(over, status):
    assert _router(**over) == status


def test_kpack_sizes():
    """The packed copy: E x row groups of MOE_KPACK_ROWS x K steps x a 36-byte block per row."""
    R = moe.MOE_KPACK_ROWS
    assert R == 256
    assert moe.moe_kpack_bytes(288, 1280, 4096) == 288 * 5 * 64 * R * 36    # exact row groups
    assert moe.moe_kpack_bytes(288, 640, 4096) == 288 * 3 * 64 * R * 36     # 640 rows: 3 groups
    assert moe.moe_kpack_bytes(288, 4096, 640) == 288 * 16 * 10 * R * 36
    assert moe.moe_kpack_bytes(1, 1, 64) == R * 36
    for bad in ((0, 64, 64), (1, 0, 64), (1, 64, 0), (1, 64, 96), (-1, 64, 64)):
        assert moe.moe_kpack_bytes(*bad) == 0


@pytest.mark.parametrize("over,status", [
    (dict(dst=0), moe.MOE_EINVAL), (dict(dst=FAKE + 4), moe.MOE_EINVAL),
    (dict(E=0), moe.MOE_EINVAL), (dict(out_f=0), moe.MOE_EINVAL), (dict(in_f=96), moe.MOE_EINVAL),
    (dict(src=_bank(FAKE + 4)), moe.MOE_EINVAL), (dict(src=_bank(0)), moe.MOE_EINVAL),
    (dict(E=4096), moe.MOE_ESHAPE), (dict(out_f=1 << 15), moe.MOE_ESHAPE),
    (dict(in_f=1 << 15), moe.MOE_ESHAPE),
])
def test_kpack_host_checks(over, status):
    a = dict(src=_bank(), E=8, out_f=256, in_f=256, dst=FAKE)
    a.update(over)
    assert moe.moe_kpack(a["src"], a["E"], a["out_f"], a["in_f"], a["dst"], stream=0,
                         raise_on_error=False) == status


def test_bank_keeps_its_tensors_alive():
    """A moe_bank stores raw addresses; bank() must hold the tensors behind them, so that a
    table or weight tensor cannot be freed (and its memory reused) while the bank is in use."""
    import gc
    import weakref

    import torch
    base = torch.zeros(4096, dtype=torch.uint8)
    s2 = torch.ones(4, dtype=torch.float32)
    tab = torch.tensor([base.data_ptr()] * 4, dtype=torch.int64)
    kp = torch.zeros(1024, dtype=torch.uint8)
    refs = [weakref.ref(t) for t in (base, s2, tab, kp)]
    b = moe.bank(base, 1024, 16, scale2=s2, experts=tab, kpack=kp)
    assert b.base == base.data_ptr() + 16 and b.experts == tab.data_ptr()
    assert b.kpack == kp.data_ptr()
    del base, s2, tab, kp
    gc.collect()
    assert all(r() is not None for r in refs)
    del b
    gc.collect()
    assert all(r() is None for r in refs)


def _layer(**over):
    a = dict(ids=FAKE, base=0, x=FAKE, topk_w=FAKE, gate=_bank(), up=_bank(), down=_bank(), T=4,
             k=2, E=8, H=256, F=64, y=FAKE, path=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(over)
    return moe.moe_layer_nvfp4(a["ids"], a["base"], a["x"], a["topk_w"], a["gate"], a["up"],
                               a["down"], a["T"], a["k"], a["E"], a["H"], a["F"], a["y"],
                               a["path"], a["ws"], a["ws_bytes"], stream=0, raise_on_error=False)


@pytest.mark.parametrize("over,status", [
    (dict(ids=0), moe.MOE_EINVAL), (dict(x=0), moe.MOE_EINVAL), (dict(y=0), moe.MOE_EINVAL),
    (dict(ws=0), moe.MOE_EINVAL), (dict(T=-1), moe.MOE_EINVAL), (dict(k=0), moe.MOE_EINVAL),
    (dict(H=96), moe.MOE_EINVAL), (dict(F=32), moe.MOE_EINVAL), (dict(path=3), moe.MOE_EINVAL),
    (dict(up=_bank(FAKE + 8)), moe.MOE_EINVAL), (dict(ws=FAKE + 64), moe.MOE_EINVAL),
    (dict(E=4096), moe.MOE_ESHAPE), (dict(T=1 << 22, k=8), moe.MOE_ESHAPE),
    (dict(ws_bytes=1024), moe.MOE_EWS), (dict(T=0), moe.MOE_OK), (dict(T=0, ids=0), moe.MOE_OK),
])
def test_layer_host_checks(over, status):
    assert _layer(**over) == status


def test_layer_workspace_covers_the_two_calls():
    for T, k, E, H, F in [(6, 10, 512, 2560, 640), (4096, 8, 288, 4096, 1280), (1, 1, 1, 64, 64)]:
        ws = moe.moe_layer_nvfp4_ws(T, k, E, H, F)
        assert ws >= moe.moe_ffn_nvfp4_ws(T, k, E, H, F) + moe.moe_route_bucket_ws(T, k, E)
        assert ws >= 4 * (E + 1 + T * k + E + 2)


@pytest.mark.parametrize("T,k,E,H,F,path", [
    (1, 10, 64, 2560, 640, moe.MOE_PATH_DECODE),       # tiny decode
    (6, 10, 512, 2560, 640, moe.MOE_PATH_DECODE),      # verify chunk
    (128, 10, 256, 2560, 640, moe.MOE_PATH_DECODE),    # E256 plateau, 5 pairs per expert
    (128, 1, 1, 2560, 320, moe.MOE_PATH_DECODE),       # shared expert: 128 tokens, one expert
    (512, 8, 288, 4096, 640, moe.MOE_PATH_DECODE),     # skewed prefill T=512: 14.2 pairs/expert
    (576, 8, 288, 4096, 640, moe.MOE_PATH_DECODE),     # 16 pairs per expert: the limit
    (577, 8, 288, 4096, 640, moe.MOE_PATH_PREFILL),    # one token past it
    (2048, 8, 288, 4096, 640, moe.MOE_PATH_PREFILL),
    (409, 10, 256, 2560, 640, moe.MOE_PATH_DECODE),    # E256 at 16 pairs per expert
    (410, 10, 256, 2560, 640, moe.MOE_PATH_PREFILL),   # one token past it
    (768, 10, 256, 2560, 640, moe.MOE_PATH_PREFILL),   # E256 at 30 pairs per expert
    (4096, 8, 288, 4096, 1280, moe.MOE_PATH_PREFILL),  # full-width prefill
    (129, 1, 1, 2560, 320, moe.MOE_PATH_PREFILL),      # past 128 tokens, 129 pairs per expert
    (6, 10, 512, 16384, 640, moe.MOE_PATH_PREFILL),    # hidden beyond the decode slices
])
def test_auto_path(T, k, E, H, F, path):
    """AUTO's rule on the host: decode for T <= 128 or at most MOE_AUTO_PAIRS_PER_EXPERT routed
    pairs per local expert, where the decode kernels can launch."""
    assert moe.moe_auto_path(T, k, E, H, F) == path


def test_auto_path_refuses_what_the_ffn_refuses():
    for args, status in [((1, 0, 8, 64, 64), moe.MOE_EINVAL), ((1, 1, 8, 96, 64), moe.MOE_EINVAL),
                         ((1, 1, 4096, 64, 64), moe.MOE_ESHAPE)]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_auto_path(*args)
        assert ei.value.status == status


def test_kpack_reference_order():
    """The GPU tests' packed-copy reference, pinned byte by byte to the header's definition: in run
    (e, g, b), slice s, byte 512 t + 8 l + j is code byte 4 + 8 (l >> 4) + j of row 32 s + 16 t +
    (l & 15), byte 1024 + 2 l + t its scale byte l >> 4; rows past the bank are zero."""
    from gpu_util import kpack_ref
    rng = np.random.default_rng(7)
    E, O, nb, R = 2, 300, 3, moe.MOE_KPACK_ROWS
    bank = rng.integers(0, 256, size=(E, O, nb * 36), dtype=np.uint8)
    out = kpack_ref(bank)
    G = -(-O // R)
    assert out.size == E * G * nb * R * 36 == moe.moe_kpack_bytes(E, O, nb * 64)
    run = R * 36
    for e in range(E):
        for g in range(G):
            for b in range(nb):
                base = ((e * G + g) * nb + b) * run
                for o in range(0, run, 7):   # every seventh byte of each run
                    s, r = divmod(o, 1152)
                    if r < 1024:
                        t, rr = divmod(r, 512)
                        l, j = divmod(rr, 8)
                        byte = 4 + 8 * (l >> 4) + j
                    else:
                        l, t = divmod(r - 1024, 2)
                        byte = l >> 4
                    row = g * R + 32 * s + 16 * t + (l & 15)
                    want = bank[e, row, b * 36 + byte] if row < O else 0
                    assert out[base + o] == want, (e, g, b, o)
