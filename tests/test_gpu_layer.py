"""The fused layer entry point (moe_layer_nvfp4: routed ids -> y in one call) against the two
calls it replaces (moe_route_bucket + moe_ffn_nvfp4) and against the fp64 oracle. On the decode
path with at most 2048 pairs and 1024 experts the decode kernels bucket the pairs themselves;
beyond that, and on the GEMM path, the bucketing kernel runs first. Every case must give y bit
for bit equal to the two calls on the same path."""
import numpy as np
import pytest
import torch

import gen
import oracle
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase, assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _layer(dc: DeviceCase, path: int) -> np.ndarray:
    ws_bytes = moe.moe_layer_nvfp4_ws(dc.T, dc.k, dc.E, dc.H, dc.F)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dc.y.fill_(float("nan"))
    moe.moe_layer_nvfp4(dc.ids, dc.base, dc.x, dc.w, dc.gate, dc.up, dc.down, dc.T, dc.k, dc.E,
                        dc.H, dc.F, dc.y, path, ws, ws_bytes)
    torch.cuda.synchronize()
    return dc.y[: dc.T].cpu().numpy()


CASES = [
    # seed, T, k, E, H, F, nonlocal fraction, expert base, fused bank
    (401, 1, 10, 64, 2560, 640, 0.0, 0, True),       # tiny decode shape
    (402, 6, 10, 512, 2560, 640, 0.0, 0, True),      # verify-chunk shape
    (403, 16, 10, 256, 2560, 640, 0.1, 3, True),     # token columns at their limit
    (404, 3, 12, 2, 512, 128, 0.0, 0, False),        # > 16 pairs per expert with token columns
    (405, 40, 8, 16, 512, 192, 0.2, 0, False),       # token chunks (> 16 tokens per expert)
    (406, 17, 4, 9, 768, 320, 0.3, 5, True),
    (407, 128, 16, 64, 256, 64, 0.1, 0, False),      # 2048 pairs: the largest in-kernel plan
    (408, 128, 20, 64, 256, 64, 0.0, 0, False),      # 2560 pairs: bucketing kernel first
    (409, 8, 4, 1500, 256, 64, 0.0, 0, False),       # 1500 experts: bucketing kernel first
    (410, 5, 3, 6, 320, 64, 0.1, 0, False),          # hidden % 256 != 0
    (412, 128, 8, 3, 256, 64, 0.0, 0, False),        # hot experts: ~340 pairs, 22 runs each
    (413, 100, 5, 2, 512, 192, 0.25, 1, True),       # hot experts beside non-local pairs
    (414, 128, 40, 8, 256, 64, 0.0, 0, False),       # 320 runs: ranges cut inside an expert
    (415, 64, 8, 32, 4096, 640, 0.1, 0, False),      # hidden 4096: one tile buffer per workgroup
    (416, 100, 12, 16, 4096, 128, 0.0, 2, True),     # the same through the bucketing kernel
]


@pytest.mark.parametrize("seed,T,k,E,H,F,frac,base,fused", CASES)
def test_layer_matches_two_calls(seed, T, k, E, H, F, frac, base, fused):
    print(f"[case] layer seed={seed} T={T} k={k} E={E} H={H} F={F} frac={frac}", flush=True)
    case = gen.make_random_case(seed, T, k, E, H, F, scales="all", nonlocal_frac=frac,
                                expert_base=base, fused=fused)
    dc = DeviceCase(case)
    ref = oracle.ffn_union(case)
    for path in (moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL, moe.MOE_PATH_AUTO):
        y2 = dc.run(path)
        y1 = _layer(dc, path)
        assert np.array_equal(y1, y2), f"fused layer differs from two calls on path {path}"
        assert_parity(y1, ref, f"layer path {path}")


# the down kernel's K split is chosen on the device from the counted experts: 4 for tiny decode
# and the 10-expert union, 2 for the 30-expert union and the shared expert, 1 for the rest
@pytest.mark.parametrize("name,T,U", [("tiny_decode", 1, None), ("verify_chunk", 6, 10),
                                      ("verify_chunk", 6, 30), ("verify_chunk", 6, 60),
                                      ("shared_expert", 128, None),
                                      ("e256_plateau", 16, None), ("e256_plateau", 128, None)])
def test_layer_workloads(name, T, U):
    print(f"[case] layer workload {name} T={T} U={U}", flush=True)
    case = gen.make_workload(name, T, U=U)
    dc = DeviceCase(case)
    y1 = _layer(dc, moe.MOE_PATH_AUTO)
    assert np.array_equal(y1, dc.run(moe.MOE_PATH_AUTO))
    assert_parity(y1, oracle.ffn_union(case), name)


def test_layer_deterministic():
    case = gen.make_random_case(411, 12, 6, 20, 512, 128, nonlocal_frac=0.1)
    dc = DeviceCase(case)
    ys = [_layer(dc, moe.MOE_PATH_DECODE) for _ in range(8)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])
