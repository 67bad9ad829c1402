"""A fixed-seed randomized sweep: random shapes (hidden 256..2560, ff 64..640, 1..64 experts,
top-k up to 12 with duplicates, 1..600 tokens), expert bases, non-local slots, both scale
distributions, fused and separate banks, second-level scales; every case through the GEMM path,
AUTO and (up to 128 tokens) the decode path against the fp64 oracle, and a quarter of them also
in the pointer-table bank form (bit for bit against the strided form)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase, assert_parity
from test_gpu_tables import _run_table_form

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _draw(rng):
    H = int(rng.choice([256, 512, 768, 1024, 1280, 2560]))
    F = int(rng.choice([64, 128, 192, 320, 384, 512, 640]))
    E = int(rng.choice([1, 2, 3, 5, 8, 17, 33, 64]))
    k = int(rng.integers(1, min(E, 10) + 1)) if rng.random() < 0.7 else int(rng.integers(1, 12))
    T = int(rng.choice([1, 2, 3, 7, 16, 17, 33, 64, 100, 128, 129, 200, 600]))
    while T * k * 3 * H * F > 4e8 and T > 1:       # keeps the fp64 oracle fast
        T = max(1, T // 2)
    while E * 3 * H * F * 36 // 64 > 60e6 and E > 1:
        E = max(1, E // 2)
    return dict(T=T, k=k, E=E, H=H, F=F, frac=float(rng.choice([0.0, 0.0, 0.1, 0.5])),
                base=int(rng.choice([0, 0, 3])), fused=bool(rng.random() < 0.5),
                scales=str(rng.choice(["all", "pow2"])), s2=bool(rng.random() < 0.3),
                table=bool(rng.random() < 0.25), seed=int(rng.integers(1, 1 << 30)))


CASES = [_draw(np.random.default_rng(20261202 + i)) for i in range(48)]


@pytest.mark.parametrize("c", CASES, ids=[f"{i}" for i in range(len(CASES))])
def test_random_case(c):
    print(f"[case] random {c}", flush=True)
    case = gen.make_random_case(c["seed"], c["T"], c["k"], c["E"], c["H"], c["F"],
                                scales=c["scales"], nonlocal_frac=c["frac"],
                                expert_base=c["base"], fused=c["fused"])
    if c["s2"]:
        case.update(gen.second_level_scales(c["seed"] + 1, c["E"]))
    ref = oracle.ffn_union(case)
    dc = DeviceCase(case)
    paths = [moe.MOE_PATH_PREFILL, moe.MOE_PATH_AUTO]
    if c["T"] <= 128:
        paths.append(moe.MOE_PATH_DECODE)
    for path in paths:
        dc.y.fill_(float("nan"))
        y = dc.run(path)
        assert np.isfinite(y).all()
        assert_parity(y, ref, f"random path {path}")
        if c["table"] and path == paths[-1]:
            assert np.array_equal(_run_table_form(dc, case, c["seed"], c["seed"] % 2 == 0, path), y)
