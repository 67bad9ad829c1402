"""Helpers for the GPU tests: upload a generated case, run the layer through the C ABI,
compare against the fp64 oracle to the parity bound."""
import numpy as np
import torch

import routed_moe_expert_amd as moe

REL_RMS_BOUND = 1e-3    # relative RMS of (y_gpu - y_oracle) over RMS(y_oracle)
MAX_ABS_BOUND = 2e-3    # max |y_gpu - y_oracle| over RMS(y_oracle)


def to_dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


class DeviceCase:
    """A generated case resident on the GPU, with every output and workspace preallocated."""

    def __init__(self, case: dict):
        self.case = case
        self.T, self.k, self.E, self.H, self.F = case["T"], case["k"], case["E"], case["H"], case["F"]
        self.base = case.get("expert_base", 0)
        P = self.T * self.k
        self.ids = to_dev(case["ids"].astype(np.int32).reshape(-1))
        self.w = to_dev(case["w"].astype(np.float32).reshape(-1))
        self.x = to_dev(case["x"])
        H, F = self.H, self.F
        rbh, rbf = H // 64 * 36, F // 64 * 36
        # optional per-expert second-level scales of each bank
        self.s2 = {key: to_dev(case[key].astype(np.float32)) if case.get(key) is not None else None
                   for key in ("gate_s2", "up_s2", "down_s2")}
        if "gate_up" in case:
            self.gu = to_dev(case["gate_up"])
            self.gate = moe.bank(self.gu, 2 * F * rbh, scale2=self.s2["gate_s2"])
            self.up = moe.bank(self.gu, 2 * F * rbh, F * rbh, scale2=self.s2["up_s2"])
        else:
            self.g = to_dev(case["gate"])
            self.u = to_dev(case["up"])
            self.gate = moe.bank(self.g, F * rbh, scale2=self.s2["gate_s2"])
            self.up = moe.bank(self.u, F * rbh, scale2=self.s2["up_s2"])
        self.d = to_dev(case["down"])
        self.down = moe.bank(self.d, H * rbf, scale2=self.s2["down_s2"])
        dev = self.ids.device
        self.offsets = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        self.pair_ids = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
        self.active = torch.empty(self.E, dtype=torch.int32, device=dev)
        self.counts = torch.empty(2, dtype=torch.int32, device=dev)
        self.bws = moe.moe_route_bucket_ws(self.T, self.k, self.E)
        self.bucket_ws = torch.empty(max(self.bws, 1), dtype=torch.uint8, device=dev)
        self.ws_bytes = moe.moe_ffn_nvfp4_ws(self.T, self.k, self.E, H, F)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.y = torch.empty(max(self.T, 1), H, dtype=torch.float32, device=dev)

    def use_kpack(self, on: bool = True):
        """Give the three banks their K-step-packed copies (moe_kpack, made once and kept), so that
        the GEMM path reads those, or go back to the row-major banks alone."""
        if not hasattr(self, "_plain"):
            g, u, d = self._plain = (self.gate, self.up, self.down)
            self._packed = (moe.with_kpack(g, self.E, self.F, self.H),
                            moe.with_kpack(u, self.E, self.F, self.H),
                            moe.with_kpack(d, self.E, self.H, self.F))
            torch.cuda.synchronize()
        self.gate, self.up, self.down = self._packed if on else self._plain

    def bucket(self, stream=None):
        moe.moe_route_bucket(self.ids, self.T, self.k, self.E, self.base, self.offsets,
                             self.pair_ids, self.active, self.counts, self.bucket_ws, self.bws,
                             stream=stream)

    def ffn(self, path=moe.MOE_PATH_AUTO, stream=None):
        moe.moe_ffn_nvfp4(self.x, self.w, self.offsets, self.pair_ids, self.active, self.counts,
                          self.gate, self.up, self.down, self.T, self.k, self.E, self.H, self.F,
                          self.y, path, self.ws, self.ws_bytes, stream=stream)

    def run(self, path=moe.MOE_PATH_AUTO):
        self.bucket()
        self.ffn(path)
        torch.cuda.synchronize()
        return self.y[: self.T].cpu().numpy()

    def bucket_result(self):
        torch.cuda.synchronize()
        return (self.offsets.cpu().numpy(), self.pair_ids.cpu().numpy()[: self.T * self.k],
                self.active.cpu().numpy(), self.counts.cpu().numpy())


def kpack_ref(bank: np.ndarray, rows: int = moe.MOE_KPACK_ROWS) -> np.ndarray:
    """The packed order from its definition: per expert, row group and K block one run; a run is
    slices of 32 rows; a slice is, for each of its two 16-row tiles, lane l = n + 16 q's code
    bytes 4 + 8 q .. 11 + 8 q of row n, then lane by lane the scale byte q of row n of tile 0 and
    of tile 1. Rows past the bank are zero."""
    E, O, rb = bank.shape
    nb, G = rb // 36, -(-O // rows)
    padded = np.zeros((E, G * rows, rb), np.uint8)
    padded[:, :O] = bank
    blk = padded.reshape(E, G, rows // 32, 2, 16, nb, 36)   # e, g, slice, tile, n, b, byte
    blk = blk.transpose(0, 1, 5, 2, 3, 4, 6)                 # e, g, b, slice, tile, n, byte
    codes = blk[..., 4:].reshape(*blk.shape[:6], 4, 8)       # ..., q, 8 bytes
    codes = codes.transpose(0, 1, 2, 3, 4, 6, 5, 7)          # e, g, b, slice, tile, q, n, 8
    scales = blk[..., :4].transpose(0, 1, 2, 3, 6, 5, 4)     # e, g, b, slice, q, n, tile
    lead = codes.shape[:4]
    out = np.concatenate([codes.reshape(*lead, 1024), scales.reshape(*lead, 128)], axis=-1)
    return out.reshape(-1)


def parity(y: np.ndarray, ref: np.ndarray):
    """(relative RMS error, max abs error / RMS(ref))."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.asarray(y, dtype=np.float64) - ref
    if rms == 0.0:
        return (0.0 if not np.any(err) else np.inf), (0.0 if not np.any(err) else np.inf)
    return float(np.sqrt(np.mean(err ** 2)) / rms), float(np.abs(err).max() / rms)


def assert_parity(y, ref, what=""):
    rel, mx = parity(y, ref)
    assert rel <= REL_RMS_BOUND and mx <= MAX_ABS_BOUND, \
        f"{what}: relRMS {rel:.3e} (bound {REL_RMS_BOUND}), max abs/RMS {mx:.3e} (bound {MAX_ABS_BOUND})"
    return rel, mx


def tile_tokens(ids: np.ndarray, E: int, expert_base: int = 0, bm: int = 128) -> np.ndarray:
    """Tokens that put every M tile of the prefill path under test: for each active expert's
    bucket (in the oracle's bucketing), cut into tiles of bm consecutive CSR pairs, the tokens of
    the tile's first pair, of the last pair of its first half, of the first pair of its second
    half and of its last pair; plus the batch's last token. Sorted, without duplicates."""
    import oracle
    ids = np.asarray(ids)
    T, k = ids.shape
    off, pairs, act, _, _ = oracle.route_bucket(ids, E, expert_base)
    tok = {T - 1}
    for e in act:
        q0, m = int(off[e]), int(off[e + 1] - off[e])
        for m0 in range(0, m, bm):
            last = min(m0 + bm, m) - 1
            for c in (m0, m0 + bm // 2 - 1, m0 + bm // 2, last):
                if m0 <= c <= last:
                    tok.add(int(pairs[q0 + c]) // k)
    return np.array(sorted(tok), dtype=np.int64)
