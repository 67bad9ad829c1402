"""The C ABI's maximum sizes on the GPU: bucketing at exactly MOE_MAX_PAIRS pairs over
MOE_MAX_EXPERTS experts (bit-exact against the oracle), and the layer at the largest hidden
(MOE_MAX_HIDDEN) and the largest ff (MOE_MAX_FF, 32 h-scale segments on the GEMM path), each
with a small other side so that the fp64 oracle stays fast. Both widths are beyond the decode
kernels' K slices, so AUTO takes the GEMM path and a forced decode path is refused."""
import numpy as np
import pytest
import torch

import gen
import oracle
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase, assert_parity

pytestmark = pytest.mark.gpu

MAX_PAIRS = 1 << 24
MAX_EXPERTS = 2048
MAX_HIDDEN = 16384
MAX_FF = 8192


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bucket_at_max_pairs():
    T, k, E, base = MAX_PAIRS // 8, 8, MAX_EXPERTS, 5
    print(f"[case] bucket max pairs T={T} k={k} E={E}", flush=True)
    rng = np.random.default_rng(111)
    ids = rng.integers(base - 3, base + E + 3, size=(T, k)).astype(np.int32)   # a few non-local
    dev = torch.device("cuda")
    d_ids = torch.from_numpy(ids.reshape(-1)).to(dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pair_ids = torch.empty(T * k, dtype=torch.int32, device=dev)
    active = torch.empty(E, dtype=torch.int32, device=dev)
    counts = torch.empty(2, dtype=torch.int32, device=dev)
    bws = moe.moe_route_bucket_ws(T, k, E)
    ws = torch.empty(max(bws, 1), dtype=torch.uint8, device=dev)
    moe.moe_route_bucket(d_ids, T, k, E, base, offsets, pair_ids, active, counts, ws, bws)
    torch.cuda.synchronize()
    r_off, r_pairs, r_act, r_nact, r_non = oracle.route_bucket(ids, E, base)
    off = offsets.cpu().numpy()
    assert np.array_equal(off, r_off)
    n_local = int(r_off[-1])
    pairs = pair_ids.cpu().numpy()
    assert np.array_equal(pairs[:n_local], r_pairs)
    flat = ids.reshape(-1).astype(np.int64) - base
    assert np.array_equal(pairs[n_local:], np.nonzero((flat < 0) | (flat >= E))[0])
    cnt = counts.cpu().numpy()
    assert cnt[0] == r_nact and cnt[1] == r_non
    assert np.array_equal(active.cpu().numpy()[:r_nact], r_act)
    # one pair more is refused before anything is enqueued
    st = moe.moe_route_bucket(d_ids, T, k + 1, E, base, offsets, pair_ids, active, counts, ws,
                              bws, raise_on_error=False)
    assert st == moe.MOE_ESHAPE


@pytest.mark.parametrize("seed,H,F", [(112, MAX_HIDDEN, 256), (113, 256, MAX_FF)])
def test_layer_at_max_width(seed, H, F):
    print(f"[case] max width H={H} F={F}", flush=True)
    case = gen.make_random_case(seed, 5, 2, 3, H, F, scales="all", nonlocal_frac=0.1)
    dc = DeviceCase(case)
    dc.bucket()
    st = moe.moe_ffn_nvfp4(dc.x, dc.w, dc.offsets, dc.pair_ids, dc.active, dc.counts, dc.gate,
                           dc.up, dc.down, dc.T, dc.k, dc.E, dc.H, dc.F, dc.y,
                           moe.MOE_PATH_DECODE, dc.ws, dc.ws_bytes, raise_on_error=False)
    assert st == moe.MOE_ESHAPE
    ref = oracle.ffn_union(case)
    y = dc.run(moe.MOE_PATH_AUTO)
    assert_parity(y, ref, f"max width H={H} F={F}")
    # the GEMM path from the K-step-packed copies at the widest K and row counts
    dc.use_kpack()
    assert np.array_equal(dc.run(moe.MOE_PATH_AUTO), y), "packed copies differ at max width"


def test_decode_pairs_beyond_lds_plan():
    """More routed pairs than the decode kernels' start-up reads into LDS (4096): the plan takes
    its pair ids from memory instead. 128 tokens x top-40 over 512 experts through AUTO."""
    print("[case] decode P>4096 T=128 k=40 E=512", flush=True)
    case = gen.make_random_case(114, 128, 40, 512, 512, 128, scales="all", nonlocal_frac=0.05)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_AUTO)
    assert_parity(y, oracle.ffn_union(case), "decode P>4096")


@pytest.mark.parametrize("path", [moe.MOE_PATH_PREFILL, moe.MOE_PATH_DECODE])
def test_tokens_beyond_grid_y_limit(path):
    """70000 tokens (more than a grid's y dimension holds): the combine loops over tokens."""
    T = 70000
    print(f"[case] T={T} path={path}", flush=True)
    case = gen.make_random_case(115, T, 1, 4, 64, 64, scales="all", nonlocal_frac=0.05)
    dc = DeviceCase(case)
    y = dc.run(path)
    tok = np.concatenate([np.arange(8), np.arange(65530, 65542), np.arange(T - 8, T)])
    assert_parity(y[tok], oracle.ffn_union(case, tokens=tok), f"T={T}")


def test_layer_at_max_pairs():
    """The whole layer (bucketing, GEMM path, combine) at exactly MOE_MAX_PAIRS routed pairs:
    2^20 tokens x top-16 over 64 experts, hidden = ff = 64; sampled tokens against the oracle."""
    T, k, E = MAX_PAIRS // 16, 16, 64
    print(f"[case] layer at max pairs T={T} k={k} E={E}", flush=True)
    case = gen.make_random_case(116, T, k, E, 64, 64, scales="all", nonlocal_frac=0.01)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_AUTO)
    tok = np.concatenate([np.random.default_rng(5).choice(T, 40, replace=False), [T - 1]])
    assert_parity(y[tok], oracle.ffn_union(case, tokens=tok), "max pairs")


@pytest.mark.parametrize("seed,T,k,E,H,F,fused", [
    (201, 5, 3, 6, 320, 64, False), (202, 24, 4, 9, 576, 192, True),
    (203, 40, 10, 32, 2624, 640, True), (204, 200, 2, 3, 64, 128, False)])
def test_hidden_multiple_of_64(seed, T, k, E, H, F, fused):
    """Hidden sizes that are multiples of 64 but not of 256 (rows not whole 16-byte chunks) on
    every path that takes them."""
    print(f"[case] hidden%64 seed={seed} T={T} k={k} E={E} H={H} F={F}", flush=True)
    case = gen.make_random_case(seed, T, k, E, H, F, scales="all", nonlocal_frac=0.1, fused=fused)
    ref = oracle.ffn_union(case)
    dc = DeviceCase(case)
    paths = [moe.MOE_PATH_PREFILL, moe.MOE_PATH_AUTO] + ([moe.MOE_PATH_DECODE] if T <= 128 else [])
    for path in paths:
        dc.y.fill_(float("nan"))
        assert_parity(dc.run(path), ref, f"H={H} path {path}")
