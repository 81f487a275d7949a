"""GPU parity of the W4A8 path with MXFP4 weights (MOE_PREC_W4A8_MX: FP8 E4M3 activations
x E2M1 codes with one E8M0 scale per 32 values along K, on the FP4 matrix cores) against
the CPU oracle.

Bars as for NVFP4: routing, tables and permuted rows bit-exact (the same code path);
expert outputs and the forward max|err| / max|ref| <= 3e-2 against the fp64 oracle; the
forward with the gather folded into GEMM1 bitwise equal to the separate entry points.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle
import token_permute_grouped_amd as tpg
from moe_synth import CONFIGS, MoeConfig, generate
from moe_synth.gen import w4a8_sweep_tokens
from tests._gpu import (DeviceProblem, assert_all_rows_written, bf16_f64, bf16_host, merged_tile_rows, rel_err, to_dev,
                        whole_tiles)

pytestmark = pytest.mark.gpu

W4A8_BAR = 3e-2
SMALL = {
    "mx_tiny": MoeConfig("mx_tiny", T=64, H=256, I=256, E=8, k=2, prec="w4a8_mx", swiglu_clamp=10.0),
    "mx_one_token": MoeConfig("mx_one_token", T=1, H=256, I=256, E=4, k=4, prec="w4a8_mx", swiglu_clamp=10.0),
    "mx_interleaved_drop": MoeConfig("mx_interleaved_drop", T=100, H=512, I=512, E=6, k=3, prec="w4a8_mx",
                                     glu_interleave=32, swiglu_clamp=10.0, drop_p=0.1),
    "mx_ragged_no_clamp": MoeConfig("mx_ragged_no_clamp", T=300, H=768, I=768, E=5, k=2, prec="w4a8_mx"),
    "mx_tight_clamp": MoeConfig("mx_tight_clamp", T=90, H=512, I=256, E=4, k=2, prec="w4a8_mx", swiglu_clamp=0.5),
    # K a multiple of 1024 and T <= 32: the persistent GEMMs with several tiles per workgroup
    "mx_persistent_il_drop": MoeConfig("mx_persistent_il_drop", T=32, H=1024, I=1024, E=64, k=8, prec="w4a8_mx",
                                       glu_interleave=32, swiglu_clamp=10.0, drop_p=0.1),
    # the single-launch forward: two token blocks per tile, interleave and drops; many small experts
    "mx_fused_t100_il_drop": MoeConfig("mx_fused_t100_il_drop", T=100, H=1024, I=1024, E=16, k=4, prec="w4a8_mx",
                                       glu_interleave=32, swiglu_clamp=10.0, drop_p=0.1),
    "mx_fused_e256": MoeConfig("mx_fused_e256", T=40, H=1024, I=2048, E=256, k=8, prec="w4a8_mx", swiglu_clamp=10.0),
    # one token, K a multiple of 512: GEMM1 split in two K halves (two workgroups per tile, partial
    # sums added by the re-quantisation); interleaved W1 and a dropped slot
    "mx_one_token_split": MoeConfig("mx_one_token_split", T=1, H=1024, I=1024, E=8, k=4, prec="w4a8_mx",
                                    glu_interleave=32, swiglu_clamp=10.0, drop_p=0.25),
    # every expert 65..85 rows: one m-tile of three 32-row token blocks each
    "mx_merged_tiles": MoeConfig("mx_merged_tiles", T=200, H=512, I=512, E=5, k=2, prec="w4a8_mx",
                                 glu_interleave=32, swiglu_clamp=10.0, drop_p=0.05),
    # k = E: every expert holds exactly T rows; 96 = the largest merged tile (three full token
    # blocks), 97 = a full 64-row tile and a 33-row one
    "mx_all_experts_96": MoeConfig("mx_all_experts_96", T=96, H=512, I=256, E=4, k=4, prec="w4a8_mx",
                                     swiglu_clamp=10.0),
    "mx_all_experts_97": MoeConfig("mx_all_experts_97", T=97, H=512, I=256, E=4, k=4, prec="w4a8_mx",
                                     swiglu_clamp=10.0),
}


@functools.lru_cache(maxsize=None)
def small(name):
    cfg = SMALL[name]
    print(f"[gpu w4a8_mx] generating {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    inp = generate(cfg, seed=0)
    return inp, DeviceProblem(inp)


@functools.lru_cache(maxsize=1)
def full_weights():
    print("[gpu w4a8_mx] generating the MXFP4 layer (H=7168 I=2048 E=32 top-8, T=256)", flush=True)
    return generate(CONFIGS["w4a8_mx"], seed=0)


def sweep_case(T: int):
    """the first T tokens of the T=256 draw"""
    base = full_weights()
    inp = dict(base, cfg=CONFIGS["w4a8_mx"].with_tokens(T), logits=base["logits"][:T], x=base["x"][:T],
               x_scale=base["x_scale"][:T])
    return inp, DeviceProblem(inp)


def _ffn_rows_err(inp, d, rows_of=None):
    cfg = inp["cfg"]
    idx, _ = d.route()
    offsets, row_src, _, x_perm, x_perm_scale = d.permute(idx)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    off = offsets.cpu().numpy()
    R = int(off[-1])
    rows = np.arange(R) if rows_of is None else rows_of(off)
    expert = np.searchsorted(off, rows, side="right") - 1
    ref = oracle.ffn_rows(inp, row_src.cpu().numpy()[rows] // cfg.k, expert)
    got = bf16_host(y)
    assert_all_rows_written(y, R, float(np.abs(ref).max()), f"{cfg.name} y_perm")
    return rel_err(bf16_f64(got[rows]), ref), got, R


@pytest.mark.parametrize("name", list(SMALL))
def test_grouped_ffn_rows(name):
    inp, d = small(name)
    err, got, R = _ffn_rows_err(inp, d)
    print(f"[gpu w4a8_mx] {name}: grouped FFN on {R} rows, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR
    assert (got[R:] == 0xFFFF).all()


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    inp, d = small(name)
    err = rel_err(bf16_f64(bf16_host(d.forward())), oracle.moe_forward(inp))
    print(f"[gpu w4a8_mx] {name}: forward, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR


@pytest.mark.parametrize("T", w4a8_sweep_tokens())
def test_forward_token_sweep(T):
    inp, d = sweep_case(T)
    out = bf16_host(d.forward())
    tokens = np.arange(T) if T <= 16 else np.unique(
        np.concatenate([np.random.default_rng(T).integers(0, T, 6), [0, T - 1]]))
    ref = oracle.moe_forward(inp, tokens)
    err = rel_err(bf16_f64(out[tokens]), ref)
    print(f"[gpu w4a8_mx] sweep T={T}: forward on {tokens.size} tokens, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR
    assert_all_rows_written(to_dev(out), T, float(np.abs(ref).max()), f"w4a8_mx T={T} forward out")


@pytest.mark.parametrize("case", list(SMALL) + ["T1", "T16", "T256"])
def test_forward_gather_in_gemm1_equals_separate_steps(case):
    inp, d = small(case) if case in SMALL else sweep_case(int(case[1:]))
    fused = bf16_host(d.forward())
    idx, w = d.route()
    offsets, _, slot_row, x_perm, x_perm_scale = d.permute(idx, canary=False)
    steps = bf16_host(d.combine(d.grouped_ffn(x_perm, x_perm_scale, offsets), slot_row, w))
    n_diff = int((fused != steps).sum())
    print(f"[gpu w4a8_mx] {case}: fused-gather forward vs separate steps, {n_diff} differing elements")
    assert n_diff == 0


def test_grouped_ffn_full_layer_sampled_rows():
    inp, d = sweep_case(256)

    def first_last(off):
        rows = []
        for e in range(inp["cfg"].E):
            if off[e + 1] > off[e]:
                rows += [off[e], off[e + 1] - 1]
        rows = np.union1d(np.array(rows, dtype=np.int64), whole_tiles(off, 64))  # + two whole 64-row m-tiles
        return np.union1d(rows, merged_tile_rows(off, 64))  # + a whole three-block (merged) m-tile

    err, got, R = _ffn_rows_err(inp, d, first_last)
    print(f"[gpu w4a8_mx] full layer: grouped FFN on the first and last row of every expert and two whole "
          f"m-tiles, max|err|/max|ref| = {err:.3e}")
    assert (got[R:] == 0xFFFF).all()
    assert err <= W4A8_BAR


@pytest.mark.parametrize("lo,hi", [(100, 160), (1, 40), (190, 225)])
def test_scales_outside_the_fp8_decoder_range_stay_exact(lo, hi):
    """block scales far outside 2^-5..2^6 (where a decode to FP8 would saturate or flush): the
    FP4 matrix cores take e2m1 * 2^s * fp8 exactly, as the oracle's definition does.  The
    global scales keep every partial sum and output finite in fp32."""
    cfg = MoeConfig("mx_wide_scales", T=40, H=512, I=256, E=4, k=2, prec="w4a8_mx", swiglu_clamp=10.0)
    inp = generate(cfg, seed=3)
    rng = np.random.default_rng(lo)
    for key, gkey in (("w1_bscale", "w1_gscale"), ("w2_bscale", "w2_gscale")):
        sc = rng.integers(lo, hi, size=inp[key].shape).astype(np.uint8)
        inp[key] = sc
        inp[gkey] = np.ldexp(np.float32(1.0), 127 - (lo + hi) // 2 - 8) * np.ones(cfg.E, np.float32)
    d = DeviceProblem(inp)
    ref = oracle.moe_forward(inp)
    assert np.isfinite(ref).all() and np.abs(ref).max() > 0
    err = rel_err(bf16_f64(bf16_host(d.forward())), ref)
    print(f"[gpu w4a8_mx] scales {lo}..{hi - 1}: forward, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR


@pytest.mark.parametrize("case", ["mx_persistent_il_drop", "mx_fused_t100_il_drop", "mx_fused_e256", "mx_one_token_split"]
                         + [f"T{T}" for T in w4a8_sweep_tokens()])
def test_single_launch_forward_equals_default(case):
    """MOE_FLAG_SINGLE_LAUNCH with MXFP4 weights: bitwise the default multi-launch forward"""
    inp, d = small(case) if case in SMALL else sweep_case(int(case[1:]))
    one = bf16_host(DeviceProblem(inp, flags=tpg.MOE_FLAG_SINGLE_LAUNCH).forward())
    n_diff = int((one != bf16_host(d.forward())).sum())
    print(f"[gpu w4a8_mx] {case}: single-launch forward vs default, {n_diff} differing elements", flush=True)
    assert n_diff == 0
