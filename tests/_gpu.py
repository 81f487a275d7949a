"""Device-side plumbing shared by the GPU tests: copies a generated workload to the
GPU and calls the library's entry points through the C ABI binding."""
from __future__ import annotations

import numpy as np
import torch

import token_permute_grouped_amd as tpg

DEV = torch.device("cuda:0")


def to_dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def bf16_host(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the bar the parity tests apply)"""
    m = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (m if m > 0 else 1.0))


def whole_tiles(offsets: np.ndarray, bm: int) -> np.ndarray:
    """every row of two whole m-tiles of bm rows: an interior tile of the largest expert and the
    first tile of the expert of median (non-zero) size"""
    counts = np.diff(offsets)
    big = int(np.argmax(counts))
    m = (int(counts[big]) // bm) // 2                      # an interior full tile where there is one
    a0 = int(offsets[big]) + m * bm
    rows = [np.arange(a0, min(a0 + bm, int(offsets[big + 1])))]
    live = np.nonzero(counts)[0]
    med = int(live[np.argsort(counts[live], kind="stable")[live.size // 2]])
    if med != big:
        rows.append(np.arange(int(offsets[med]), min(int(offsets[med]) + bm, int(offsets[med + 1]))))
    return np.concatenate(rows).astype(np.int64)


def merged_tile_rows(offsets: np.ndarray, bm: int) -> np.ndarray:
    """every row of the last m-tile of the largest expert whose rows end in a remainder of 1..bm/2
    after at least one full tile (the W4A8 tile list merges that remainder into the tile before it,
    a tile of up to 1.5 bm rows); empty if no expert has one"""
    counts = np.diff(offsets)
    ok = (counts > bm) & (counts % bm >= 1) & (counts % bm <= bm // 2)
    if not ok.any():
        return np.zeros(0, dtype=np.int64)
    e = int(np.argmax(np.where(ok, counts, -1)))
    start = int(offsets[e]) + (int(counts[e]) // bm - 1) * bm
    return np.arange(start, int(offsets[e + 1]), dtype=np.int64)


def assert_all_rows_written(dev_bits, n_rows: int, ref_absmax: float, what: str):
    """no element of the first n_rows rows still holds the 0xFFFF fill (a bf16 NaN), and the largest
    magnitude stays within 4x of the sampled reference's (a skipped GEMM1 tile would leave the
    workspace fill in h and blow the row up)"""
    live = dev_bits[:n_rows]
    n_canary = int((live == -1).sum())
    assert n_canary == 0, f"{what}: {n_canary} elements never written"
    amax = float((live.to(torch.int32) << 16).view(torch.float32).abs().max())
    assert np.isfinite(amax) and amax <= 4.0 * ref_absmax, (what, amax, ref_absmax)


class DeviceProblem:
    """One workload resident on the GPU, plus the output and workspace buffers of each call."""

    def __init__(self, inp: dict, flags: int = 0):
        self.inp = inp
        cfg = self.cfg = inp["cfg"]
        self.w4 = cfg.prec != "bf16"
        self.p = tpg.make_problem(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, tpg.PRECISIONS[cfg.prec],
                                  cfg.glu_interleave, cfg.swiglu_clamp, flags)
        self.logits = to_dev(inp["logits"])
        self.drop = to_dev(inp.get("slot_drop"))
        self.x = to_dev(inp["x"])
        self.x_scale = to_dev(inp.get("x_scale"))
        self.w = {k: to_dev(inp.get(k)) for k in ("w1", "w1_bscale", "w1_gscale", "w2", "w2_bscale", "w2_gscale")}
        self.weights = tpg.make_weights(self.w["w1"], self.w["w2"], self.w["w1_bscale"], self.w["w1_gscale"],
                                        self.w["w2_bscale"], self.w["w2_gscale"])
        self.S = cfg.T * cfg.k

    def workspace(self, which, fill=None):
        n = tpg.moe_call_workspace_bytes(self.p, which)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        if fill is not None:
            ws.fill_(fill)
        return ws

    # ---------------------------------------------------------------- steps
    def route(self):
        cfg = self.cfg
        idx = torch.full((cfg.T, cfg.k), 0x7FFFFFFF, dtype=torch.int32, device=DEV)
        w = torch.full((cfg.T, cfg.k), float("nan"), dtype=torch.float32, device=DEV)
        tpg.moe_route_topk(self.logits, self.drop, self.p, idx, w)
        return idx, w

    def permute(self, topk_idx, canary=True):
        cfg = self.cfg
        S = self.S
        offsets = torch.full((cfg.E + 1,), 0x7FFFFFFF, dtype=torch.int32, device=DEV)
        row_src = torch.full((S,), 0x7FFFFFFF, dtype=torch.int32, device=DEV)
        slot_row = torch.full((S,), 0x7FFFFFFF, dtype=torch.int32, device=DEV)
        if self.w4:
            x_perm = torch.full((S, cfg.H), 0x7F, dtype=torch.uint8, device=DEV)
            x_perm_scale = torch.full((S, cfg.H // 128), float("nan"), dtype=torch.float32, device=DEV)
        else:
            x_perm = torch.full((S, cfg.H), -1, dtype=torch.int16, device=DEV)  # 0xFFFF: a bf16 NaN
            x_perm_scale = None
        ws = self.workspace(tpg.MOE_WS_PERMUTE, fill=0xAB if canary else None)
        tpg.moe_permute(self.x, self.x_scale, topk_idx, self.p, offsets, row_src, slot_row, x_perm, x_perm_scale, ws)
        return offsets, row_src, slot_row, x_perm, x_perm_scale

    def grouped_ffn(self, x_perm, x_perm_scale, offsets, ws=None):
        cfg = self.cfg
        y = torch.full((self.S, cfg.H), -1, dtype=torch.int16, device=DEV)
        if ws is None:
            ws = self.workspace(tpg.MOE_WS_GROUPED_FFN, fill=0xCD)
        tpg.moe_grouped_ffn(x_perm, x_perm_scale, offsets, self.weights, self.p, y, ws)
        return y

    def combine(self, y_perm, slot_row, topk_w):
        cfg = self.cfg
        out = torch.full((cfg.T, cfg.H), -1, dtype=torch.int16, device=DEV)
        tpg.moe_unpermute_combine(y_perm, slot_row, topk_w, self.p, out)
        return out

    def forward(self, ws=None):
        cfg = self.cfg
        out = torch.full((cfg.T, cfg.H), -1, dtype=torch.int16, device=DEV)
        if ws is None:
            ws = self.workspace(tpg.MOE_WS_FORWARD, fill=0xEF)
        tpg.moe_forward(self.logits, self.drop, self.x, self.x_scale, self.weights, self.p, out, ws)
        return out
