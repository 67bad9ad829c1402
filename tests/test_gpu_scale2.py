"""Two-level NVFP4 (per-expert fp32 second-level scales per bank) on both paths against the
fp64 oracle, fused and separate banks, small cases and workload-size cases."""
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


@pytest.mark.parametrize("seed,T,k,E,H,F,fused,banks", [
    (61, 5, 4, 6, 512, 128, False, ("gate_s2", "up_s2", "down_s2")),
    (62, 40, 3, 9, 256, 192, True, ("gate_s2", "up_s2", "down_s2")),
    (63, 17, 2, 5, 768, 1344, False, ("down_s2",)),          # KS > 1 down reduction
    (64, 33, 8, 12, 256, 64, True, ("up_s2",)),
])
def test_scale2_small(seed, T, k, E, H, F, fused, banks):
    print(f"[case] scale2 seed={seed} T={T} k={k} E={E} H={H} F={F} fused={fused} {banks}",
          flush=True)
    case = gen.make_random_case(seed, T, k, E, H, F, fused=fused, nonlocal_frac=0.1)
    case.update(gen.second_level_scales(seed + 1, E, banks))
    ref = oracle.ffn_union(case)
    dc = DeviceCase(case)
    for path, name in ((moe.MOE_PATH_DECODE, "decode"), (moe.MOE_PATH_PREFILL, "prefill")):
        assert_parity(dc.run(path), ref, "scale2 " + name)


@pytest.mark.parametrize("name,T,path,n_check", [("e256_plateau", 32, moe.MOE_PATH_DECODE, 8),
                                                 ("skewed_prefill", 512, moe.MOE_PATH_PREFILL, 8)])
def test_scale2_workloads(name, T, path, n_check):
    print(f"[case] scale2 workload {name} T={T}", flush=True)
    case = gen.make_workload(name, T)
    case.update(gen.second_level_scales(65, case["E"]))
    dc = DeviceCase(case)
    y = dc.run(path)
    tok = np.random.default_rng(T).choice(T, size=n_check, replace=False)
    tok[0] = T - 1
    assert_parity(y[tok], oracle.ffn_per_slot(case, tokens=tok), name)
