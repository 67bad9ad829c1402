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
    assert_parity(dc.run(moe.MOE_PATH_AUTO), ref, f"max width H={H} F={F}")
