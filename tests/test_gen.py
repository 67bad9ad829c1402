"""The seeded input generator (CPU only)."""
import numpy as np
import pytest
import torch

import gen


def _skew_cdf(e, E, a=1.35):
    """P(expert <= e) under expert = min(floor(u^a * E), E - 1), u uniform: u^a < (e+1)/E."""
    return np.minimum(((np.asarray(e, dtype=np.float64) + 1) / E) ** (1 / a), 1.0)


def test_route_skewed_is_a_function_of_the_pair():
    """Each pair's expert depends on its index only: a shorter batch is a prefix of a longer one,
    and other seeds give other routings."""
    a = gen.route_skewed(512, 8, 288).reshape(-1)
    b = gen.route_skewed(4096, 8, 288).reshape(-1)
    assert np.array_equal(a, b[: a.size])
    assert not np.array_equal(a, gen.route_skewed(512, 8, 288, seed=1).reshape(-1))
    assert a.min() >= 0 and b.max() <= 287


def test_route_skewed_closed_form_hot_expert():
    """P(expert 0) = P(u^1.35 < 1/E) = (1/E)^(1/1.35), about 4.34 times the mean load at E=288."""
    ids = gen.route_skewed(4096, 8, 288).reshape(-1)
    p0 = (1 / 288) ** (1 / 1.35)
    n = ids.size
    assert abs((ids == 0).sum() - n * p0) < 4 * np.sqrt(n * p0)
    assert abs(288 * p0 - 4.34) < 0.01


def test_route_skewed_follows_the_power_law():
    """Chi-square of the per-expert counts against the closed-form bin probabilities
    P(e) = ((e+1)/E)^(1/1.35) - (e/E)^(1/1.35) (the last bin takes the rest): far inside the
    tail at 287 degrees of freedom (mean 287, sd 24)."""
    E, n = 288, 4096 * 8
    ids = gen.route_skewed(4096, 8, E).reshape(-1)
    cdf = _skew_cdf(np.arange(E), E)
    p = np.diff(np.concatenate([[0.0], cdf]))
    p[-1] = 1.0 - cdf[-2]
    obs = np.bincount(ids, minlength=E)
    chi2 = ((obs - n * p) ** 2 / (n * p)).sum()
    assert chi2 < 287 + 6 * 24
    # a wrong exponent is caught: the same counts against a = 1.58 (an 8x hot expert)
    p8 = np.diff(np.concatenate([[0.0], _skew_cdf(np.arange(E), E, 1.58)]))
    assert ((obs - n * p8) ** 2 / (n * p8)).sum() > 287 + 20 * 24


@pytest.mark.parametrize("U", [10, 30, 60])
def test_route_union(U):
    ids, w = gen.make_routing("verify_chunk", 6, U=U)
    assert ids.shape == (6, 10)
    assert np.unique(ids).size == U
    assert all(np.unique(r).size == 10 for r in ids)
    assert np.all(np.bincount(ids.reshape(-1), minlength=512)[np.unique(ids)] == 60 // U)


def test_route_cyclic_all_active_from_32():
    for T, U in [(16, 160), (32, 256), (128, 256)]:
        ids, _ = gen.make_routing("e256_plateau", T)
        assert np.unique(ids).size == U
        assert all(np.unique(r).size == 10 for r in ids)


def test_route_distinct():
    ids, _ = gen.make_routing("tiny_decode", 3)
    assert all(np.unique(r).size == 10 for r in ids) and ids.max() < 64


def test_router_weights_softmax_rows():
    w = gen.router_weights(3, 50, 8)
    assert w.dtype == np.float32 and np.all(w > 0)
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() < 1e-6


def test_bank_scale_distributions():
    b = gen.nvfp4_bank(1, 1, 2, 4, 128, scales="pow2").reshape(-1, 36)
    s = b[:, :4]
    assert np.all(s % 8 == 0) and s.min() >= 0x08 and s.max() <= 0x48
    assert set(np.unique(s)) == {8 * e for e in range(1, 10)}
    b = gen.nvfp4_bank(1, 1, 8, 64, 256, scales="all").reshape(-1, 36)
    assert b[:, :4].max() <= 0x7E and np.unique(b[:, :4]).size == 127
    # code bytes are uniform: both nibbles take all 16 values
    c = b[:, 4:]
    assert np.unique(c & 15).size == 16 and np.unique(c >> 4).size == 16


def test_bf16_rounding_is_rne():
    vals = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], dtype=np.float32)
    got = gen.f32_to_bf16_bits(vals)
    ref = torch.tensor(vals).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(got, ref)
    x = gen.bf16_normal(1, (4, 256))
    xf = torch.tensor(x.astype(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(xf.mean()) < 0.2 and 0.8 < xf.std() < 1.2


def test_streams_are_independent_and_reproducible():
    a = gen.make_workload("tiny_decode", 1, with_banks=False)
    b = gen.make_workload("tiny_decode", 1, with_banks=False)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["ids"], b["ids"])
    c = gen.make_workload("tiny_decode", 1, seed=9, with_banks=False)
    assert not np.array_equal(a["x"], c["x"])


def test_route_union_rotated_disjoint_windows():
    a = gen.route_union_rotated(2, 6, 10, 512, 60, 0)
    b = gen.route_union_rotated(2, 6, 10, 512, 60, 1)
    assert np.unique(a).size == 60 and np.unique(b).size == 60
    assert np.intersect1d(a, b).size == 0
    assert all(np.unique(r).size == 10 for r in a)
