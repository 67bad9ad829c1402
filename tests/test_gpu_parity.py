"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bucketing must match bit for bit; the FFN output must be within relRMS <= 1e-3 and
max abs <= 2e-3 * RMS(y) of the oracle; repeated calls must be bit-identical.
"""
import hashlib

import numpy as np
import pytest
import torch

import gen
import oracle
import routed_moe_expert_amd as moe
from gpu_util import DeviceCase, assert_parity, tile_tokens

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _print_case(tag, **kw):
    print(f"[case] {tag} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _check_bucket(dc: DeviceCase):
    case = dc.case
    off, pairs, act, cnt = dc.bucket_result()
    r_off, r_pairs, r_act, r_nact, r_non = oracle.route_bucket(case["ids"], dc.E, dc.base)
    assert np.array_equal(off, r_off)
    n_local = int(r_off[-1])
    assert np.array_equal(pairs[:n_local], r_pairs)
    flat = case["ids"].reshape(-1).astype(np.int64) - dc.base
    nonlocal_pairs = np.nonzero((flat < 0) | (flat >= dc.E))[0]
    assert np.array_equal(pairs[n_local:], nonlocal_pairs)
    assert cnt[0] == r_nact and cnt[1] == r_non
    assert np.array_equal(act[:r_nact], r_act)


# ----------------------------------------------------------------------------------- bucketing

@pytest.mark.parametrize("T,k,E,base,frac", [
    (1, 10, 64, 0, 0.0), (6, 10, 512, 0, 0.0), (7, 3, 5, 0, 0.0), (50, 4, 16, 100, 0.3),
    (9, 2, 1, 0, 0.0), (200, 8, 288, 0, 0.5), (1000, 8, 2048, 0, 0.1), (3, 4, 7, 0, 1.0),
    (0, 4, 8, 0, 0.0), (513, 2, 3, 0, 0.0),
    # around and past the single-workgroup limit (4096 pairs): chunked histogram/scan/scatter
    (512, 8, 64, 0, 0.0), (4097, 1, 7, 3, 0.2), (4096, 8, 288, 0, 0.0), (3000, 6, 2048, 0, 0.3)])
def test_bucket_random(T, k, E, base, frac):
    _print_case("bucket_random", T=T, k=k, E=E, base=base, frac=frac)
    case = gen.make_random_case(T * 7 + k + E, T, k, E, 256, 64, nonlocal_frac=frac,
                                expert_base=base)
    dc = DeviceCase(case)
    dc.bucket()
    _check_bucket(dc)


@pytest.mark.parametrize("name,T,U", [("tiny_decode", 1, None), ("verify_chunk", 6, 10),
                                      ("verify_chunk", 6, 60), ("e256_plateau", 128, None),
                                      ("skewed_prefill", 512, None), ("skewed_prefill", 4096, None)])
def test_bucket_workloads(name, T, U):
    _print_case("bucket_workload", name=name, T=T, U=U)
    w = gen.WORKLOADS[name]
    ids, wts = gen.make_routing(name, T, U)
    case = dict(T=T, k=w["k"], E=w["E"], H=256, F=64, ids=ids, w=wts,
                x=np.zeros((T, 256), np.uint16), gate=np.zeros((w["E"], 64, 144), np.uint8),
                up=np.zeros((w["E"], 64, 144), np.uint8), down=np.zeros((w["E"], 256, 36), np.uint8))
    dc = DeviceCase(case)
    dc.bucket()
    _check_bucket(dc)


# ----------------------------------------------------------------------------- FFN: decode path

SMALL = [
    # seed, T, k, E, H, F, scales, nonlocal fraction, expert base, fused
    (1, 1, 1, 1, 256, 64, "all", 0.0, 0, False),
    (2, 5, 2, 3, 256, 128, "all", 0.0, 0, True),
    (3, 17, 4, 8, 512, 192, "all", 0.2, 5, False),
    (4, 40, 2, 2, 256, 64, "pow2", 0.0, 0, False),     # > 8 tokens per expert: token chunks
    (5, 3, 6, 4, 768, 128, "all", 0.5, 0, True),       # duplicates within tokens
    (6, 12, 3, 16, 256, 320, "all", 0.0, 0, False),
    # the down kernel's K split taken on the device, from its smallest to a wider one: ff 576
    # (9 blocks: slices of 9 or 5), ff 1280 (20 blocks: from 2 slices of 10 to 4 of 5), ff 2560
    # (40 blocks: 4 slices of 10, no wider), each with a union of a few experts
    (7, 2, 3, 64, 512, 576, "all", 0.0, 0, False),
    (8, 3, 2, 32, 1024, 1280, "all", 0.1, 0, True),
    (9, 2, 2, 8, 256, 2560, "all", 0.0, 0, False),
]


@pytest.mark.parametrize("seed,T,k,E,H,F,scales,frac,base,fused", SMALL)
def test_decode_small(seed, T, k, E, H, F, scales, frac, base, fused):
    _print_case("decode_small", seed=seed, T=T, k=k, E=E, H=H, F=F, frac=frac)
    case = gen.make_random_case(seed, T, k, E, H, F, scales=scales, nonlocal_frac=frac,
                                expert_base=base, fused=fused)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_DECODE)
    _check_bucket(dc)
    ref = oracle.ffn_union(case)
    assert_parity(y, ref, "decode_small")


_WL = {}


def _workload(name, T, U=None):
    key = (name, T, U)
    if key not in _WL:
        _WL.clear()
        _WL[key] = gen.make_workload(name, T, U=U)
    return _WL[key]


@pytest.mark.parametrize("name,T,U", [
    ("tiny_decode", 1, None), ("verify_chunk", 6, 10), ("verify_chunk", 6, 30),
    ("verify_chunk", 6, 60), ("e256_plateau", 16, None), ("e256_plateau", 32, None),
    ("e256_plateau", 64, None), ("e256_plateau", 80, None), ("e256_plateau", 128, None),
    ("skewed_prefill", 16, None), ("full_prefill", 8, None)])
def test_decode_workloads(name, T, U):
    """Every decode workload at full size through AUTO (the decode path at these T), every token
    compared with the oracle."""
    _print_case("decode_workload", name=name, T=T, U=U)
    case = _workload(name, T, U)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_AUTO)
    _check_bucket(dc)
    assert_parity(y, oracle.ffn_union(case), name)


@pytest.mark.parametrize("F,U", [(640, 10), (640, 30), (1280, 10)])
def test_decode_union_split(F, U):
    """A union of a few experts in a routing that could hold many (60 pairs over 64 experts): the
    host sizes the down kernel for the widest union (one K slice at ff 640, two at ff 1280) and
    the kernel widens its K split once its plan has counted the experts (4 slices for 10 experts,
    2 for 30). Every token against the oracle."""
    _print_case("decode_union_split", F=F, U=U)
    case = gen.make_random_case(500 + U + F, 6, 10, 64, 2560, F, fused=(F == 640))
    case["ids"] = gen.route_union(500 + U, 6, 10, 64, U).astype(np.int32)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_DECODE)
    _check_bucket(dc)
    assert_parity(y, oracle.ffn_union(case), "decode_union_split")


def test_decode_beyond_slice_width_uses_gemm_path():
    """hidden = 5376 is wider than the decode kernels' K slices: forcing decode is refused with
    MOE_ESHAPE, and AUTO computes the layer on the GEMM path."""
    case = gen.make_random_case(34, 3, 2, 3, 5376, 64)
    dc = DeviceCase(case)
    dc.bucket()
    st = moe.moe_ffn_nvfp4(dc.x, dc.w, dc.offsets, dc.pair_ids, dc.active, dc.counts, dc.gate,
                           dc.up, dc.down, dc.T, dc.k, dc.E, dc.H, dc.F, dc.y,
                           moe.MOE_PATH_DECODE, dc.ws, dc.ws_bytes, raise_on_error=False)
    assert st == moe.MOE_ESHAPE
    y = dc.run(moe.MOE_PATH_AUTO)
    assert_parity(y, oracle.ffn_union(case), "auto wide hidden")


def test_decode_deterministic():
    case = gen.make_random_case(31, 24, 4, 6, 512, 128, nonlocal_frac=0.1)
    dc = DeviceCase(case)
    hashes = set()
    for _ in range(10):
        y = dc.run(moe.MOE_PATH_DECODE)
        hashes.add(hashlib.sha256(y.tobytes()).hexdigest())
    assert len(hashes) == 1


def test_tokens_without_local_slots_get_zero():
    case = gen.make_random_case(32, 6, 3, 4, 256, 64)
    ids = case["ids"].copy()
    ids[2, :] = 77              # token 2: every slot on another rank
    ids[4, :] = -5
    case["ids"] = ids
    dc = DeviceCase(case)
    dc.y.fill_(np.nan)
    y = dc.run(moe.MOE_PATH_DECODE)
    assert np.all(y[2] == 0) and np.all(y[4] == 0)
    assert_parity(y, oracle.ffn_union(case), "nonlocal rows")


def test_zero_tokens_is_noop():
    case = gen.make_random_case(33, 0, 2, 3, 256, 64)
    dc = DeviceCase(case)
    dc.bucket()
    off, _, _, cnt = dc.bucket_result()
    assert np.all(off == 0) and np.all(cnt == 0)
    assert moe.moe_ffn_nvfp4(dc.x, dc.w, dc.offsets, dc.pair_ids, dc.active, dc.counts, dc.gate,
                             dc.up, dc.down, 0, 2, 3, 256, 64, dc.y, 0, dc.ws, dc.ws_bytes) == moe.MOE_OK


# ---------------------------------------------------------------------------- FFN: prefill path

PREFILL_SMALL = [
    # seed, T, k, E, H, F, scales, nonlocal fraction, expert base, fused
    (11, 3, 2, 4, 256, 64, "all", 0.0, 0, False),
    (12, 150, 2, 2, 256, 128, "all", 0.0, 0, True),      # > 128 pairs per expert: several M tiles
    (13, 70, 4, 9, 512, 192, "all", 0.3, 2, False),
    (14, 40, 8, 5, 768, 64, "pow2", 0.0, 0, False),      # duplicates within tokens
    (15, 300, 1, 1, 256, 320, "all", 0.0, 0, False),     # one expert, 300 pairs: ragged last tile
]


@pytest.mark.parametrize("seed,T,k,E,H,F,scales,frac,base,fused", PREFILL_SMALL)
def test_prefill_small(seed, T, k, E, H, F, scales, frac, base, fused):
    _print_case("prefill_small", seed=seed, T=T, k=k, E=E, H=H, F=F, frac=frac)
    case = gen.make_random_case(seed, T, k, E, H, F, scales=scales, nonlocal_frac=frac,
                                expert_base=base, fused=fused)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_PREFILL)
    assert_parity(y, oracle.ffn_union(case), "prefill_small")


# pairs per expert on each side of the GEMMs' column steps: gate/up runs 32, 64, 96 or 128 token
# columns of a 128-pair M tile, down 16, 32, 48 or 64 of a 64-pair half tile
COLUMN_COUNTS = [1, 15, 16, 17, 32, 33, 48, 49, 64, 65, 96, 97, 127, 128, 129, 192, 255]


@pytest.mark.parametrize("F", [320, 512])
def test_prefill_column_cases(F):
    """Experts whose pair counts sit at and beside every column step of both GEMMs, every token
    compared, on both gate/up kernels (ff 320: 128-feature N tiles, 512: 256-feature ones), from
    the row-major banks and, bit for bit the same, from the K-step-packed copies."""
    E, T = len(COLUMN_COUNTS), sum(COLUMN_COUNTS)
    _print_case("prefill_column_cases", T=T, E=E, F=F)
    case = gen.make_random_case(61, T, 1, E, 512, F)
    perm = np.random.default_rng(61).permutation(T)
    case["ids"] = np.repeat(np.arange(E, dtype=np.int32), COLUMN_COUNTS)[perm].reshape(T, 1)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_PREFILL)
    assert_parity(y, oracle.ffn_union(case), f"column cases ff {F}")
    dc.use_kpack(True)
    assert np.array_equal(dc.run(moe.MOE_PATH_PREFILL), y), "packed copies differ"


@pytest.mark.parametrize("name,T", [("skewed_prefill", 512), ("skewed_prefill", 2048),
                                    ("skewed_prefill", 4096), ("full_prefill", 4096)])
def test_prefill_workloads(name, T):
    """Full-size prefill workloads. The GEMM path (forced) on the tokens that cover every M tile:
    each tile's first and last pair and both ends of its halves. AUTO must give what the path
    moe_auto_path names gives, bit for bit; where that is the decode path (skewed T=512: 14 pairs
    per expert), it is compared on every token."""
    _print_case("prefill_workload", name=name, T=T)
    case = _workload(name, T)
    dc = DeviceCase(case)
    y = dc.run(moe.MOE_PATH_PREFILL)
    _check_bucket(dc)
    tok = tile_tokens(case["ids"], dc.E)
    auto = moe.moe_auto_path(T, dc.k, dc.E, dc.H, dc.F)
    if auto == moe.MOE_PATH_DECODE:
        ref = oracle.ffn_union(case)
        assert_parity(y[tok], ref[tok], name + " gemm path")
        yd = dc.run(moe.MOE_PATH_DECODE)
        assert_parity(yd, ref, name + " decode path")
        assert np.array_equal(dc.run(moe.MOE_PATH_AUTO), yd), "AUTO differs from the decode path"
    else:
        print(f"[case] comparing {tok.size} tokens", flush=True)
        assert_parity(y[tok], oracle.ffn_union(case, tokens=tok), name)
        assert np.array_equal(dc.run(moe.MOE_PATH_AUTO), y), "AUTO differs from the GEMM path"


def test_e256_forced_through_gemm_path():
    """The E256 decode shape forced through the GEMM path, every token compared."""
    case = _workload("e256_plateau", 128)
    dc = DeviceCase(case)
    assert_parity(dc.run(moe.MOE_PATH_PREFILL), oracle.ffn_union(case), "e256 gemm path")


def test_prefill_deterministic_and_matches_decode():
    case = gen.make_random_case(41, 64, 4, 6, 512, 128, nonlocal_frac=0.1)
    dc = DeviceCase(case)
    hashes = set()
    for _ in range(5):
        y = dc.run(moe.MOE_PATH_PREFILL)
        hashes.add(hashlib.sha256(y.tobytes()).hexdigest())
    assert len(hashes) == 1
    yd = dc.run(moe.MOE_PATH_DECODE)
    ref = oracle.ffn_union(case)
    assert_parity(y, ref, "prefill")
    assert_parity(yd, ref, "decode")
