"""The shared expert (one dense SwiGLU expert over all T rows) on the routed kernels: parity with
the fp64 oracle on both paths, and the pages' split-versus-full check (the ff dimension split in
two shards whose outputs add up to the full expert's)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase, assert_parity, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("T,H,F", [(1, 2560, 320), (16, 2560, 320), (128, 2560, 320),
                                   (37, 512, 384), (600, 2560, 320), (17, 512, 192),
                                   (32, 512, 192), (33, 256, 64)])
def test_shared_expert_matches_oracle(T, H, F):
    print(f"[case] shared T={T} H={H} F={F}", flush=True)
    case = gen.make_shared_case(300 + T, T, H, F)
    ref = oracle.ffn_union(case)
    dc = DeviceCase(case)
    paths = [moe.MOE_PATH_AUTO, moe.MOE_PATH_PREFILL] + ([moe.MOE_PATH_DECODE] if T <= 128 else [])
    for path in paths:
        assert_parity(dc.run(path), ref, f"shared path {path}")


@pytest.mark.parametrize("T,F,F1", [(16, 320, 192), (128, 384, 192), (600, 320, 128)])
def test_shared_expert_split_vs_full(T, F, F1):
    """Two ff shards (as two tensor-parallel ranks would hold them) summed against the full
    expert: each within the parity bound of the oracle, and their sum within it of the full
    expert's GPU output."""
    print(f"[case] shared split T={T} F={F} F1={F1}", flush=True)
    case = gen.make_shared_case(400 + T, T, 2560, F)
    a, b = gen.split_ff(case, F1)
    y = DeviceCase(case).run()
    ya, yb = DeviceCase(a).run(), DeviceCase(b).run()
    assert_parity(y, oracle.ffn_union(case), "full")
    assert_parity(ya + yb, y, "shards summed vs full")
    rel, mx = parity(ya + yb, y)
    print(f"[split] relRMS {rel:.2e} max abs/RMS {mx:.2e}", flush=True)


@pytest.mark.parametrize("T,G", [(128, 8), (100, 7), (16, 16)])
def test_shared_expert_virtual_experts(T, G):
    """The shared expert as G virtual experts (tokens dealt round-robin, every virtual expert's
    rows at the one weight copy through pointer tables) computes the one-expert layer bit for bit
    on both paths: a token column's sums do not depend on which tokens share its tile."""
    print(f"[case] shared virtual T={T} G={G}", flush=True)
    case = gen.make_shared_case(500 + T, T, 2560, 320)
    dc = DeviceCase(case)
    ids, w = gen.shared_virtual_routing(T, G)
    dv = DeviceCase(dict(case, E=G, ids=ids, w=w))
    # dv's strided banks would address G experts in a one-expert allocation: replace them before
    # any call with tables whose G entries all point at the one expert's rows
    tabs = [torch.full((G,), b.base, dtype=torch.int64, device="cuda")
            for b in (dv.gate, dv.up, dv.down)]
    dv.gate, dv.up, dv.down = (moe.bank(None, 0, experts=tb) for tb in tabs)
    ref = oracle.ffn_union(case)
    for path in (moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL):
        y1 = dc.run(path)
        yv = dv.run(path)
        assert np.array_equal(yv, y1), f"virtual experts differ on path {path}"
        assert_parity(yv, ref, f"shared virtual path {path}")
