"""The layer captured in a HIP graph: the library's launches hold no memset and no allocation,
so a captured call replays. Every replay, with other eager work between the replays, must give y
bit for bit equal to the eager call, on both paths and in both call forms."""
import numpy as np
import pytest
import torch

import gen
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _layer_call(dc, ws, ws_bytes, path, stream):
    moe.moe_layer_nvfp4(dc.ids, dc.base, dc.x, dc.w, dc.gate, dc.up, dc.down, dc.T, dc.k, dc.E,
                        dc.H, dc.F, dc.y, path, ws, ws_bytes, stream=stream)


def _two_calls(dc, path, stream):
    dc.bucket(stream=stream)
    dc.ffn(path, stream=stream)


@pytest.mark.parametrize("form", ["layer", "two_calls"])
@pytest.mark.parametrize("seed,T,k,E,H,F,path", [
    (601, 6, 10, 64, 512, 128, moe.MOE_PATH_DECODE),
    (602, 40, 8, 6, 512, 192, moe.MOE_PATH_DECODE),     # experts of several 16-pair runs
    (603, 96, 4, 16, 256, 128, moe.MOE_PATH_PREFILL),
])
def test_graph_replay_matches_eager(form, seed, T, k, E, H, F, path):
    print(f"[case] graph {form} seed={seed} T={T} k={k} E={E} path={path}", flush=True)
    case = gen.make_random_case(seed, T, k, E, H, F, nonlocal_frac=0.1)
    dc = DeviceCase(case)
    other = DeviceCase(gen.make_random_case(seed + 50, T, k, E, H, F))
    ws_bytes = moe.moe_layer_nvfp4_ws(T, k, E, H, F)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def call(stream):
        if form == "layer":
            _layer_call(dc, ws, ws_bytes, path, stream)
        else:
            _two_calls(dc, path, stream)

    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = dc.y[:T].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        other.run(path)            # eager work on other buffers between the replays
        dc.y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc.y[:T], ref), f"replay {rep} differs from the eager call"
    del g
