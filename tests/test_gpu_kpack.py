"""The K-step-packed weight copy (moe_kpack) and the GEMM path reading it. The copy must hold the
row-major bank's 36-byte blocks in the order the header defines, bit for bit, and y computed from
the packed copies must equal y from the row-major banks bit for bit: the GEMM feeds the same
operands to the same MFMA lanes, only staged from contiguous runs in another order, and does the
same arithmetic."""
import numpy as np
import pytest
import torch

import gen
import oracle
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase, assert_parity, kpack_ref, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("E,O,K,table", [(3, 256, 512, False), (2, 640, 320, False),
                                         (5, 100, 64, False), (4, 320, 1280, True)])
def test_kpack_layout(E, O, K, table):
    print(f"[case] kpack layout E={E} O={O} K={K} table={table}", flush=True)
    bank = gen.nvfp4_bank(40 + E, gen.S_GATE, E, O, K, "all")
    dev = to_dev(bank)
    rb = K // 64 * 36
    if table:   # experts in reverse order through a pointer table
        tab = torch.tensor([dev.data_ptr() + (E - 1 - e) * O * rb for e in range(E)],
                           dtype=torch.int64, device="cuda")
        src, ref = moe.bank(None, 0, experts=tab), kpack_ref(bank[::-1])
    else:
        src, ref = moe.bank(dev, O * rb), kpack_ref(bank)
    dst = torch.full((moe.moe_kpack_bytes(E, O, K),), 0xAB, dtype=torch.uint8, device="cuda")
    assert dst.numel() == ref.size
    moe.moe_kpack(src, E, O, K, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), ref)


def _layer(dc: DeviceCase, path: int) -> np.ndarray:
    ws_bytes = moe.moe_layer_nvfp4_ws(dc.T, dc.k, dc.E, dc.H, dc.F)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    moe.moe_layer_nvfp4(dc.ids, dc.base, dc.x, dc.w, dc.gate, dc.up, dc.down, dc.T, dc.k, dc.E,
                        dc.H, dc.F, dc.y, path, ws, ws_bytes)
    torch.cuda.synchronize()
    return dc.y[: dc.T].cpu().numpy()


CASES = [
    # seed, T, k, E, H, F, nonlocal fraction, expert base, fused gate_up bank
    (61, 40, 4, 8, 512, 640, 0.1, 0, False),     # ff 640: the last gate/up row group half full
    (62, 300, 6, 12, 320, 192, 0.0, 2, True),    # hidden 320: down rows past one group; fused
    (63, 200, 8, 16, 1024, 256, 0.2, 0, False),  # whole row groups
]


@pytest.mark.parametrize("seed,T,k,E,H,F,frac,base,fused", CASES)
def test_prefill_kpack_bitwise(seed, T, k, E, H, F, frac, base, fused):
    print(f"[case] kpack prefill seed={seed} T={T} k={k} E={E} H={H} F={F}", flush=True)
    case = gen.make_random_case(seed, T, k, E, H, F, scales="all", nonlocal_frac=frac,
                                expert_base=base, fused=fused)
    dc = DeviceCase(case)
    y0, d0 = dc.run(moe.MOE_PATH_PREFILL), dc.run(moe.MOE_PATH_DECODE)
    dc.use_kpack()
    y1 = dc.run(moe.MOE_PATH_PREFILL)
    assert np.array_equal(y0, y1), "GEMM path from the packed copies differs"
    assert np.array_equal(_layer(dc, moe.MOE_PATH_PREFILL), y1), "one-call layer differs"
    assert np.array_equal(dc.run(moe.MOE_PATH_DECODE), d0), "the decode path must ignore kpack"
    assert_parity(y1, oracle.ffn_union(case), "prefill from packed copies")


@pytest.mark.parametrize("name,T", [("skewed_prefill", 4096), ("full_prefill", 4096)])
def test_prefill_workload_kpack_bitwise(name, T):
    """Full size: every token equal bit for bit to the row-major banks' GEMM path, which
    test_prefill_workloads compares with the oracle."""
    print(f"[case] kpack workload {name} T={T}", flush=True)
    dc = DeviceCase(gen.make_workload(name, T))
    y0 = dc.run(moe.MOE_PATH_PREFILL)
    dc.use_kpack()
    assert np.array_equal(dc.run(moe.MOE_PATH_PREFILL), y0)
