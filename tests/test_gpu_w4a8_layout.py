"""GPU checks of the tiled W4A8 weight layout (MOE_W4_LAYOUT_TILED).

moe_w4a8_tile_weights must regroup the bytes exactly as include/moe.h defines (compared
with a numpy regrouping of the same arrays, bit for bit, NVFP4 nibbles included), and a
forward or grouped FFN on tiled weights must give bitwise the output of the same call on
row-major weights (the GEMMs see the same values in the same order; only their addresses,
and for NVFP4 the dequant's path to K order, change).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import token_permute_grouped_amd as tpg
from moe_synth import CONFIGS, MoeConfig, generate
from tests._gpu import DEV, DeviceProblem, bf16_host, to_dev

pytestmark = pytest.mark.gpu


def split_nibbles_host(codes: np.ndarray) -> np.ndarray:
    """NVFP4 codes of every 4-byte group (byte i = codes 2i, 2i + 1, low nibble first) regrouped so
    that byte i holds codes i (low nibble) and i + 4 (high nibble)"""
    g = codes.reshape(-1, 4)
    k = np.stack([g & 15, g >> 4], axis=-1).reshape(-1, 8)  # the eight codes in K order
    return (k[:, :4] | (k[:, 4:] << 4)).astype(np.uint8).reshape(codes.shape)


def tile_host(codes: np.ndarray, bscale: np.ndarray, bs: int):
    """the layout's definition (include/moe.h), element by element: every 32-row block's 256-wide
    piece is one run; code granule g of row r at 1024 (2 q + t) + 16 (32 h + r) with g = 4 q + 2 h
    + t; scale byte j of row r at 8 (32 h + r) + 4 q + u (j = 8 q + 4 h + u, NVFP4) or 4 (32 h + r)
    + 2 q + u (j = 4 q + 2 h + u, MXFP4); NVFP4 codes (bs = 16) with their nibbles regrouped per
    4-byte group"""
    E, N, Kh = codes.shape
    nc, per = Kh // 128, 256 // bs
    src_c = split_nibbles_host(codes) if bs == 16 else codes
    out_c = np.zeros(E * N * Kh, dtype=np.uint8)
    out_s = np.zeros(bscale.size, dtype=np.uint8)
    for e in range(E):
        for row in range(N):
            blk, r = e * (N // 32) + row // 32, row % 32
            for c in range(nc):
                piece = (blk * nc + c) * 4096
                for g in range(8):
                    q, h, t = g // 4, (g // 2) % 2, g % 2
                    d = piece + 1024 * (2 * q + t) + 16 * (32 * h + r)
                    out_c[d:d + 16] = src_c[e, row, 128 * c + 16 * g:128 * c + 16 * g + 16]
                spiece = (blk * nc + c) * 32 * per
                for j in range(per):
                    if bs == 16:
                        q, h, u = j // 8, (j // 4) % 2, j % 4
                        d = 8 * (32 * h + r) + 4 * q + u
                    else:
                        q, h, u = j // 4, (j // 2) % 2, j % 2
                        d = 4 * (32 * h + r) + 2 * q + u
                    out_s[spiece + d] = bscale[e, row, per * c + j]
    return out_c.reshape(codes.shape), out_s.reshape(bscale.shape)


def tile_device(codes: torch.Tensor, bscale: torch.Tensor, prec: int):
    E, N, Kh = codes.shape
    ct, st = torch.empty_like(codes), torch.empty_like(bscale)
    tpg.moe_w4a8_tile_weights(codes, bscale, ct, st, E, N, 2 * Kh, prec)
    return ct, st


@pytest.mark.parametrize("prec,shape", [("w4a8", (3, 64, 512)), ("w4a8_mx", (3, 64, 512)),
                                        ("w4a8", (2, 96, 1280)), ("w4a8_mx", (1, 32, 256)),
                                        ("w4a8_mx", (5, 160, 768))])
def test_tile_weights_regroups_bytes_exactly(prec, shape):
    E, N, K = shape
    bs = 32 if prec == "w4a8_mx" else 16
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    bscale = rng.integers(0, 256, size=(E, N, K // bs), dtype=np.uint8)
    ct, st = tile_device(to_dev(codes), to_dev(bscale), tpg.PRECISIONS[prec])
    want_c, want_s = tile_host(codes, bscale, bs)
    assert np.array_equal(ct.cpu().numpy(), want_c)
    assert np.array_equal(st.cpu().numpy(), want_s)


CASES = {
    "nv_tiny": MoeConfig("nv_tiny", T=64, H=256, I=256, E=8, k=2, prec="w4a8", swiglu_clamp=10.0),
    "mx_interleaved_drop": MoeConfig("mx_interleaved_drop", T=100, H=512, I=512, E=6, k=3, prec="w4a8_mx",
                                     glu_interleave=32, swiglu_clamp=10.0, drop_p=0.1),
    "nv_ragged": MoeConfig("nv_ragged", T=300, H=768, I=768, E=5, k=2, prec="w4a8"),
    # persistent GEMMs (T <= 32, K a multiple of 1024), several tiles per workgroup
    "nv_persistent": MoeConfig("nv_persistent", T=32, H=1024, I=1024, E=64, k=8, prec="w4a8",
                               glu_interleave=32, swiglu_clamp=10.0),
    "mx_persistent": MoeConfig("mx_persistent", T=16, H=1024, I=1024, E=32, k=8, prec="w4a8_mx",
                               swiglu_clamp=10.0),
    # one token: GEMM1 in two K halves (the dequant of the tiled nibble order in the split form)
    "nv_one_token_split": MoeConfig("nv_one_token_split", T=1, H=1024, I=1024, E=8, k=4, prec="w4a8",
                                    glu_interleave=32, swiglu_clamp=10.0, drop_p=0.25),
    # two token blocks per tile in the single-launch forward
    "nv_fused_t100": MoeConfig("nv_fused_t100", T=100, H=1024, I=1024, E=16, k=4, prec="w4a8", swiglu_clamp=10.0,
                               drop_p=0.1),
    # above 128 tokens: two- and three-block tiles, with H = 4096 and 20-24 one-tile experts more
    # tiles (640-768) than two workgroups per CU
    "nv_t200_three_block": MoeConfig("nv_t200_three_block", T=200, H=512, I=1024, E=5, k=2, prec="w4a8",
                                          swiglu_clamp=10.0, drop_p=0.05),
    "mx_t256_h4096": MoeConfig("mx_t256_h4096", T=256, H=4096, I=1024, E=24, k=4, prec="w4a8_mx",
                                    glu_interleave=32),
    "nv_t200_h4096": MoeConfig("nv_t200_h4096", T=200, H=4096, I=1024, E=20, k=4, prec="w4a8",
                                    swiglu_clamp=10.0, drop_p=0.1),
}


def _tiled_problem(inp):
    """a DeviceProblem whose weights are the tiled copies of inp's"""
    cfg = inp["cfg"]
    d = DeviceProblem(inp)
    prec = tpg.PRECISIONS[cfg.prec]
    w = dict(d.w)
    w["w1"], w["w1_bscale"] = tile_device(d.w["w1"], d.w["w1_bscale"], prec)
    w["w2"], w["w2_bscale"] = tile_device(d.w["w2"], d.w["w2_bscale"], prec)
    d.w_tiled = w
    d.weights = tpg.make_weights(w["w1"], w["w2"], w["w1_bscale"], w["w1_gscale"], w["w2_bscale"], w["w2_gscale"],
                                 tpg.MOE_W4_LAYOUT_TILED)
    return d


@pytest.mark.parametrize("name", list(CASES))
def test_forward_and_grouped_ffn_on_tiled_weights_equal_row_major(name):
    cfg = CASES[name]
    print(f"[gpu w4 layout] {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} {cfg.prec}", flush=True)
    inp = generate(cfg, seed=0)
    rows, tiled = DeviceProblem(inp), _tiled_problem(inp)
    assert (bf16_host(rows.forward()) == bf16_host(tiled.forward())).all()
    idx, _ = rows.route()
    offsets, _, _, x_perm, x_perm_scale = rows.permute(idx)
    y_rows = bf16_host(rows.grouped_ffn(x_perm, x_perm_scale, offsets))
    y_tiled = bf16_host(tiled.grouped_ffn(x_perm, x_perm_scale, offsets))
    R = int(offsets[-1].item())
    assert (y_rows[:R] == y_tiled[:R]).all()


# every GEMM form on the full layer in both formats: the K-split GEMM1 (T = 1), the persistent
# GEMMs (T = 16), one- and two-block tiles above 32 tokens (T = 64, 128), three-block tiles (T = 256)
@pytest.mark.parametrize("wl,T", [("w4a8", 1), ("w4a8", 16), ("w4a8", 64), ("w4a8", 256), ("w4a8_mx", 1),
                                  ("w4a8_mx", 16), ("w4a8_mx", 128), ("w4a8_mx", 256)])
def test_full_layer_forward_on_tiled_weights_equals_row_major(wl, T):
    print(f"[gpu w4 layout] {wl} layer T={T}", flush=True)
    inp = generate(CONFIGS[wl], seed=0, T=T)
    rows, tiled = DeviceProblem(inp), _tiled_problem(inp)
    a, b = bf16_host(rows.forward()), bf16_host(tiled.forward())
    torch.cuda.synchronize()
    assert (a == b).all()


@pytest.mark.parametrize("name", ["nv_persistent", "nv_one_token_split", "nv_fused_t100", "mx_persistent"])
def test_single_launch_forward_on_tiled_weights_equals_row_major(name):
    """the single-launch kernel on tiled weights (for NVFP4 its dequant of the tiled nibble order, in
    the one-block, two-block and K-halves forms) against the default forward on row-major weights"""
    cfg = CASES[name]
    print(f"[gpu w4 layout] single launch {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} {cfg.prec}",
          flush=True)
    inp = generate(cfg, seed=0)
    rows, tiled = DeviceProblem(inp), _tiled_problem(inp)
    tiled.p.flags = tpg.MOE_FLAG_SINGLE_LAUNCH
    assert (bf16_host(rows.forward()) == bf16_host(tiled.forward())).all()
