"""moe_ffn_nvfp4_static (workspace in the library's own device array, no allocation) against
moe_ffn_nvfp4 with a caller-allocated workspace: the same kernels, so the outputs must be equal
bit for bit. Two calls in a row, the second on a smaller input, on both paths; then a size
beyond the array is refused before anything is enqueued."""
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


def _static(dc: DeviceCase, path: int) -> np.ndarray:
    dc.bucket()
    dc.y.fill_(float("nan"))
    moe.moe_ffn_nvfp4_static(dc.x, dc.w, dc.offsets, dc.pair_ids, dc.active, dc.counts, dc.gate,
                             dc.up, dc.down, dc.T, dc.k, dc.E, dc.H, dc.F, dc.y, path)
    torch.cuda.synchronize()
    return dc.y[: dc.T].cpu().numpy()


@pytest.mark.parametrize("path", [moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL, moe.MOE_PATH_AUTO])
def test_static_workspace_matches_caller_workspace(path):
    big = gen.make_random_case(301, 96, 10, 64, 2560, 640, scales="all", nonlocal_frac=0.1,
                               fused=True)
    small = gen.make_random_case(302, 5, 4, 9, 512, 192, scales="all", nonlocal_frac=0.1)
    for case, tag in ((big, "first, larger"), (small, "second, smaller")):
        print(f"[case] static ws path={path} {tag} T={case['T']} k={case['k']} E={case['E']}",
              flush=True)
        dc = DeviceCase(case)
        y_static = _static(dc, path)
        y_ref = dc.run(path)
        assert np.array_equal(y_static, y_ref), f"static workspace differs ({tag})"
        tok = np.arange(min(case["T"], 8))
        assert_parity(y_static[tok], oracle.ffn_union(case, tokens=tok), f"static {tag}")


def test_static_workspace_too_small_is_refused():
    T, k, E, H, F = 4096, 8, 288, 4096, 1280
    assert moe.moe_ffn_nvfp4_ws(T, k, E, H, F) > moe.MOE_STATIC_WS_BYTES
    x = torch.empty(1, dtype=torch.int16, device="cuda")
    b = moe.bank(x, 0)
    st = moe.moe_ffn_nvfp4_static(x, x, x, x, x, x, b, b, b, T, k, E, H, F, x, 0,
                                  raise_on_error=False)
    assert st == moe.MOE_EWS
