"""Banks in the per-expert pointer-table form (moe_bank.experts) against the same banks in the
strided form and against the fp64 oracle, on both paths.

The table form only changes where a workgroup finds an expert's rows, so y must match the strided
form bit for bit. The experts are stored out of order and at unrelated addresses: one device
allocation per expert (small cases), or a permuted copy of the bank with a gap between experts."""
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


def _table_copy(bank: np.ndarray, seed: int, separate: bool, keep: list) -> torch.Tensor:
    """Device int64 [E] of addresses of expert e's rows, stored away from the strided layout.
    Every device tensor involved (the copies and the table) is appended to `keep`: a moe_bank
    holds raw addresses, so they must outlive the call."""
    E = bank.shape[0]
    if separate:
        addrs = []
        for e in range(E):
            t = torch.from_numpy(np.ascontiguousarray(bank[e]).view(np.int8).reshape(-1)).cuda()
            keep.append(t)
            addrs.append(t.data_ptr())
    else:
        perm = np.random.default_rng(seed).permutation(E)
        per = bank[0].nbytes
        pitch = per + 256                         # a gap between experts
        buf = torch.zeros(E * pitch, dtype=torch.int8, device="cuda")
        keep.append(buf)
        for slot, e in enumerate(perm):
            buf[slot * pitch: slot * pitch + per] = torch.from_numpy(
                np.ascontiguousarray(bank[e]).view(np.int8).reshape(-1)).cuda()
        where = np.empty(E, np.int64)
        where[perm] = np.arange(E)
        addrs = [buf.data_ptr() + int(where[e]) * pitch for e in range(E)]
    assert all(a % 16 == 0 for a in addrs)
    tab = torch.tensor(addrs, dtype=torch.int64, device="cuda")
    keep.append(tab)   # the bank holds only the table's address: keep it alive for the call
    return tab


def _run_table_form(dc: DeviceCase, case: dict, seed: int, separate: bool, path: int):
    keep = []
    F, H = dc.F, dc.H
    rbh = H // 64 * 36
    s2 = dc.s2
    if "gate_up" in case:
        tab = _table_copy(case["gate_up"], seed, separate, keep)
        gate = moe.bank(None, 0, scale2=s2["gate_s2"], experts=tab)
        up_tab = tab + F * rbh                    # up rows follow the gate rows of each expert
        keep.append(up_tab)
        up = moe.bank(None, 0, scale2=s2["up_s2"], experts=up_tab)
    else:
        gate = moe.bank(None, 0, scale2=s2["gate_s2"],
                        experts=_table_copy(case["gate"], seed, separate, keep))
        up = moe.bank(None, 0, scale2=s2["up_s2"],
                      experts=_table_copy(case["up"], seed + 1, separate, keep))
    down = moe.bank(None, 0, scale2=s2["down_s2"],
                    experts=_table_copy(case["down"], seed + 2, separate, keep))
    dc.bucket()
    dc.y.fill_(np.nan)
    moe.moe_ffn_nvfp4(dc.x, dc.w, dc.offsets, dc.pair_ids, dc.active, dc.counts, gate, up, down,
                      dc.T, dc.k, dc.E, dc.H, dc.F, dc.y, path, dc.ws, dc.ws_bytes)
    torch.cuda.synchronize()
    return dc.y[: dc.T].cpu().numpy()


@pytest.mark.parametrize("seed,T,k,E,H,F,fused,separate,s2", [
    (101, 5, 3, 6, 512, 128, False, True, False),
    (102, 24, 4, 9, 256, 192, True, True, True),
    (103, 6, 10, 64, 2560, 640, True, False, False),      # verify-chunk shapes, permuted bank
    (104, 40, 2, 4, 768, 1344, False, True, True),        # down K split over waves; chunks
])
@pytest.mark.parametrize("path", [moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL])
def test_pointer_table_matches_strided(seed, T, k, E, H, F, fused, separate, s2, path):
    print(f"[case] tables seed={seed} T={T} k={k} E={E} H={H} F={F} fused={fused} "
          f"separate={separate} s2={s2} path={path}", flush=True)
    case = gen.make_random_case(seed, T, k, E, H, F, scales="all", nonlocal_frac=0.1, fused=fused)
    if s2:
        case.update(gen.second_level_scales(seed + 5, E))
    dc = DeviceCase(case)
    y_strided = dc.run(path)
    y_table = _run_table_form(dc, case, seed, separate, path)
    assert np.array_equal(y_table, y_strided), "table form differs from strided form"
    tok = np.random.default_rng(seed).choice(T, size=min(T, 6), replace=False)
    tok[0] = T - 1
    assert_parity(y_table[tok], oracle.ffn_per_slot(case, tokens=tok), "pointer table")
