"""GPU parity of the router step (moe_router_topk) against the fp64 oracle: expert ids bit-exact
(both sides select on the same fp32 logits), weights to fp32 rounding; then router -> bucket ->
FFN end to end against the oracle chain."""
import hashlib

import numpy as np
import pytest
import torch

import gen
import oracle
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase, assert_parity, to_dev

pytestmark = pytest.mark.gpu

# fp32 softmax against fp64: exp of an fp32 difference (|l_j - l_0| < ~10 here), an fp32 sum of
# k terms and one division stay well inside 1e-5 relative
W_RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_router(logits, k):
    T, E = logits.shape
    lg = to_dev(logits)
    ids = torch.full((max(T, 1), k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((max(T, 1), k), -1.0, dtype=torch.float32, device="cuda")
    moe.moe_router_topk(lg, T, E, k, ids, w)
    torch.cuda.synchronize()
    return ids[:T].cpu().numpy(), w[:T].cpu().numpy()


@pytest.mark.parametrize("T,E,k,ties", [
    (1, 64, 10, False), (6, 512, 10, True), (128, 256, 10, True), (4096, 288, 8, False),
    (4096, 288, 8, True), (33, 33, 33, True), (5, 2048, 64, True), (7, 65, 1, True),
    (301, 100, 7, True), (3, 1, 1, False), (9, 130, 64, False)])
def test_router_matches_oracle(T, E, k, ties):
    print(f"[case] router T={T} E={E} k={k} ties={ties}", flush=True)
    logits = gen.router_logits(1000 + E + k, T, E, ties=ties)
    ids, w = _run_router(logits, k)
    r_ids, r_w = oracle.router_topk(logits, k)
    assert np.array_equal(ids, r_ids)
    assert np.allclose(w, r_w, rtol=W_RTOL, atol=0)


def test_router_zero_tokens_is_noop():
    lg = torch.zeros(1, 8, dtype=torch.float32, device="cuda")
    ids = torch.full((1, 2), -7, dtype=torch.int32, device="cuda")
    w = torch.full((1, 2), -7.0, dtype=torch.float32, device="cuda")
    moe.moe_router_topk(lg, 0, 8, 2, ids, w)
    torch.cuda.synchronize()
    assert torch.all(ids == -7) and torch.all(w == -7.0)


def test_router_deterministic():
    logits = gen.router_logits(7, 2048, 512, ties=True)
    hashes = set()
    for _ in range(4):
        ids, w = _run_router(logits, 10)
        hashes.add(hashlib.sha256(ids.tobytes() + w.tobytes()).hexdigest())
    assert len(hashes) == 1


def test_router_bucket_ffn_chain():
    """Logits -> moe_router_topk -> moe_route_bucket -> moe_ffn_nvfp4 (both paths), against the
    oracle router feeding the oracle FFN."""
    T, E, k, H, F = 37, 24, 4, 256, 128
    print(f"[case] router chain T={T} E={E} k={k} H={H} F={F}", flush=True)
    case = gen.make_random_case(77, T, k, E, H, F)
    logits = gen.router_logits(78, T, E)
    r_ids, r_w = oracle.router_topk(logits, k)
    ids, w = _run_router(logits, k)
    assert np.array_equal(ids, r_ids)
    ref = oracle.ffn_union(dict(case, ids=r_ids, w=r_w.astype(np.float32)))
    dc = DeviceCase(dict(case, ids=ids, w=w))
    for path, name in ((moe.MOE_PATH_DECODE, "decode"), (moe.MOE_PATH_PREFILL, "prefill")):
        assert_parity(dc.run(path), ref, "router chain " + name)
