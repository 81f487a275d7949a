"""GPU parity of the W4A8 path (FP8 E4M3 activations x NVFP4 weights dequantised
to FP8 in-kernel) against the CPU oracle.

Bars: the NVFP4 -> FP8 dequant of every (code, block scale) pair bit-exact in both
nibble positions; routing, tables and permuted rows (fp8 codes and their fp32
scales) bit-exact; expert outputs and the forward max|err| / max|ref| <= 3e-2
against the fp64 oracle (the kernel accumulates in fp32 and re-quantises the
SwiGLU output from fp32 values, so a few fp8 codes of h may land one step away
from the oracle's).
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import token_permute_grouped_amd as tpg
from moe_synth import CONFIGS, MoeConfig, generate
from moe_synth.gen import w4a8_sweep_tokens
from tests._gpu import DEV, DeviceProblem, assert_all_rows_written, bf16_f64, bf16_host, merged_tile_rows, rel_err, \
    to_dev, whole_tiles

pytestmark = pytest.mark.gpu

W4A8_BAR = 3e-2
SMALL = {
    "w4_tiny": MoeConfig("w4_tiny", T=64, H=256, I=256, E=8, k=2, prec="w4a8", swiglu_clamp=10.0),
    "w4_one_token": MoeConfig("w4_one_token", T=1, H=256, I=256, E=4, k=4, prec="w4a8", swiglu_clamp=10.0),
    "w4_interleaved_drop": MoeConfig("w4_interleaved_drop", T=100, H=512, I=512, E=6, k=3, prec="w4a8",
                                     glu_interleave=32, swiglu_clamp=10.0, drop_p=0.1),
    "w4_ragged_no_clamp": MoeConfig("w4_ragged_no_clamp", T=300, H=768, I=768, E=5, k=2, prec="w4a8"),
    "w4_tight_clamp": MoeConfig("w4_tight_clamp", T=90, H=512, I=256, E=4, k=2, prec="w4a8", swiglu_clamp=0.5),
    # K a multiple of 1024 and T <= 32: the persistent GEMMs, ~1000 GEMM1 blocks over the grid (several
    # tiles per workgroup, each next tile's first chunks prefetched), interleave-32 and dropped slots
    "w4_persistent_il_drop": MoeConfig("w4_persistent_il_drop", T=32, H=1024, I=1024, E=64, k=8, prec="w4a8",
                                       glu_interleave=32, swiglu_clamp=10.0, drop_p=0.1),
    # the single-launch forward (H, I multiples of 1024, at most 256 tokens and 2048 slots): two
    # token blocks per tile, interleave and drops; and many small experts (m-tiles of a few rows)
    "w4_fused_t100_il_drop": MoeConfig("w4_fused_t100_il_drop", T=100, H=1024, I=1024, E=16, k=4, prec="w4a8",
                                       glu_interleave=32, swiglu_clamp=10.0, drop_p=0.1),
    "w4_fused_e256": MoeConfig("w4_fused_e256", T=40, H=1024, I=2048, E=256, k=8, prec="w4a8", swiglu_clamp=10.0),
    # one token, K = 1024: GEMM1 split in two K halves (two workgroups per tile, partial sums added by
    # the re-quantisation)
    "w4_one_token_split": MoeConfig("w4_one_token_split", T=1, H=1024, I=512, E=8, k=4, prec="w4a8",
                                    swiglu_clamp=10.0),
    # every expert 65..85 rows: one m-tile of three 32-row token blocks each (a remainder of at most
    # 32 rows joins the expert's 64-row tile), one of them with a single extra row
    "w4_merged_tiles": MoeConfig("w4_merged_tiles", T=200, H=512, I=512, E=5, k=2, prec="w4a8",
                                 glu_interleave=32, swiglu_clamp=10.0, drop_p=0.05),
    # k = E: every expert holds exactly T rows; 96 = the largest merged tile (three full token
    # blocks), 97 = a full 64-row tile and a 33-row one
    "w4_all_experts_96": MoeConfig("w4_all_experts_96", T=96, H=512, I=256, E=4, k=4, prec="w4a8",
                                     swiglu_clamp=10.0),
    "w4_all_experts_97": MoeConfig("w4_all_experts_97", T=97, H=512, I=256, E=4, k=4, prec="w4a8",
                                     swiglu_clamp=10.0),
}


@functools.lru_cache(maxsize=None)
def small(name):
    cfg = SMALL[name]
    print(f"[gpu w4a8] generating {name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    inp = generate(cfg, seed=0)
    return inp, DeviceProblem(inp)


@functools.lru_cache(maxsize=1)
def full_weights():
    print("[gpu w4a8] generating the W4A8 layer (H=7168 I=2048 E=32 top-8, T=256)", flush=True)
    return generate(CONFIGS["w4a8"], seed=0)


def sweep_case(T: int):
    """the first T tokens of the T=256 draw (the generator's x and logits rows do not depend on T)"""
    base = full_weights()
    inp = dict(base, cfg=CONFIGS["w4a8"].with_tokens(T), logits=base["logits"][:T], x=base["x"][:T],
               x_scale=base["x_scale"][:T])
    return inp, DeviceProblem(inp)


def test_dequant_table_every_nibble_position_bit_exact():
    out = torch.full((8, 16, 256), 0x55, dtype=torch.uint8, device=DEV)
    tpg.moe_w4a8_dequant_table(out)
    got = out.cpu().numpy()
    ref = oracle.fp4_to_fp8_table()
    for p in range(8):
        want = ref[(np.arange(16) + p) % 16]
        bad = np.argwhere(got[p] != want)
        assert bad.size == 0, f"position {p}: first mismatches (c, scale) {bad[:8].tolist()}"


@pytest.mark.parametrize("name", list(SMALL))
def test_permute_fp8_rows_and_scales_bit_exact(name):
    inp, d = small(name)
    cfg = inp["cfg"]
    idx, _ = d.route()
    offsets, row_src, slot_row, x_perm, x_perm_scale = d.permute(idx)
    torch.cuda.synchronize()
    ref_idx, _ = oracle.route(inp["logits"], cfg.k, inp.get("slot_drop"))
    assert (idx.cpu().numpy() == ref_idx).all()
    _, ref_off, ref_rs, ref_sr = oracle.tables(ref_idx, cfg.E)
    assert (offsets.cpu().numpy() == ref_off).all()
    assert (slot_row.cpu().numpy() == ref_sr).all()
    R = int(ref_off[-1])
    tok = ref_rs[:R] // cfg.k
    assert (x_perm.cpu().numpy()[:R] == inp["x"][tok]).all()
    xs = x_perm_scale.cpu().numpy()
    assert (xs[:R].view(np.uint32) == inp["x_scale"][tok].view(np.uint32)).all()
    assert (x_perm.cpu().numpy()[R:] == 0x7F).all()      # canary rows past R untouched


@pytest.mark.parametrize("name", list(SMALL))
def test_grouped_ffn_rows(name):
    inp, d = small(name)
    cfg = inp["cfg"]
    idx, _ = d.route()
    offsets, row_src, _, x_perm, x_perm_scale = d.permute(idx)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    R = int(off[-1])
    rows = np.arange(R)
    expert = np.searchsorted(off, rows, side="right") - 1
    ref = oracle.ffn_rows(inp, row_src.cpu().numpy()[rows] // cfg.k, expert)
    got_bits = bf16_host(y)
    err = rel_err(bf16_f64(got_bits[rows]), ref)
    print(f"[gpu w4a8] {name}: grouped FFN on {R} rows, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR
    assert (got_bits[R:] == 0xFFFF).all()


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    inp, d = small(name)
    out = bf16_host(d.forward())
    ref = oracle.moe_forward(inp)
    err = rel_err(bf16_f64(out), ref)
    print(f"[gpu w4a8] {name}: forward, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR


@pytest.mark.parametrize("T", w4a8_sweep_tokens())
def test_forward_token_sweep(T):
    inp, d = sweep_case(T)
    out = bf16_host(d.forward())
    tokens = np.arange(T) if T <= 16 else np.unique(
        np.concatenate([np.random.default_rng(T).integers(0, T, 6), [0, T - 1]]))
    ref = oracle.moe_forward(inp, tokens)
    err = rel_err(bf16_f64(out[tokens]), ref)
    print(f"[gpu w4a8] sweep T={T}: forward on {tokens.size} tokens, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR
    assert_all_rows_written(to_dev(out), T, float(np.abs(ref).max()), f"w4a8 T={T} forward out")


@pytest.mark.parametrize("case", list(SMALL) + ["T1", "T16", "T256"])
def test_forward_gather_in_gemm1_equals_separate_steps(case):
    """the W4A8 forward reads the fp8 rows and their scales through row_src inside GEMM1 instead
    of gathering x_perm first; its output must be bitwise what the separate entry points give"""
    inp, d = small(case) if case in SMALL else sweep_case(int(case[1:]))
    fused = bf16_host(d.forward())
    idx, w = d.route()
    offsets, row_src, slot_row, x_perm, x_perm_scale = d.permute(idx, canary=False)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    steps = bf16_host(d.combine(y, slot_row, w))
    n_diff = int((fused != steps).sum())
    print(f"[gpu w4a8] {case}: fused-gather forward vs separate steps, {n_diff} differing elements")
    assert n_diff == 0


def test_grouped_ffn_full_layer_sampled_rows():
    inp, d = sweep_case(256)
    cfg = inp["cfg"]
    idx, _ = d.route()
    offsets, row_src, _, x_perm, x_perm_scale = d.permute(idx)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    rows = []
    for e in range(cfg.E):
        if off[e + 1] > off[e]:
            rows += [off[e], off[e + 1] - 1]
    rows = np.union1d(np.array(rows, dtype=np.int64), whole_tiles(off, 64))  # + two whole 64-row m-tiles
    rows = np.union1d(rows, merged_tile_rows(off, 64))  # + a whole three-block (merged) m-tile
    expert = np.searchsorted(off, rows, side="right") - 1
    ref = oracle.ffn_rows(inp, row_src.cpu().numpy()[rows] // cfg.k, expert)
    err = rel_err(bf16_f64(bf16_host(y)[rows]), ref)
    print(f"[gpu w4a8] full layer: grouped FFN on {rows.size} rows, max|err|/max|ref| = {err:.3e}")
    assert err <= W4A8_BAR
    R = int(off[-1])
    assert_all_rows_written(y, R, float(np.abs(ref).max()), "w4a8 T=256 y_perm")
    assert (bf16_host(y)[R:] == 0xFFFF).all()


def _fused_words(ws):
    """(go, next_item, done, err) of the single-launch forward's hand-off block (workspace offset 0,
    one word per 128-byte line)"""
    b = ws[:512].cpu().numpy()
    return (int(b[:8].view(np.uint64)[0]), *(int(b[o:o + 4].view(np.uint32)[0]) for o in (128, 256, 384)))


def single_launch(inp):
    return DeviceProblem(inp, flags=tpg.MOE_FLAG_SINGLE_LAUNCH)


@pytest.mark.parametrize("case", ["w4_persistent_il_drop", "w4_fused_t100_il_drop", "w4_fused_e256"]
                         + [f"T{T}" for T in w4a8_sweep_tokens()])
def test_single_launch_forward_equals_default(case):
    """MOE_FLAG_SINGLE_LAUNCH: the whole forward in one persistent launch, bitwise the default
    multi-launch forward (and within the bar of the oracle through it)"""
    inp, d = small(case) if case in SMALL else sweep_case(int(case[1:]))
    one = bf16_host(single_launch(inp).forward())
    n_diff = int((one != bf16_host(d.forward())).sum())
    print(f"[gpu w4a8] {case}: single-launch forward vs default, {n_diff} differing elements", flush=True)
    assert n_diff == 0


@pytest.mark.parametrize("T", [1, 16, 100, 256])
def test_single_launch_forward_leaves_its_words_clean(T):
    """after the single-launch forward: the go word reset, no bounded wait gave up, every workgroup
    counted out, every item claimed; the same workspace then serves another token count"""
    inp, d0 = sweep_case(T)
    d = single_launch(inp)
    ws = d.workspace(tpg.MOE_WS_FORWARD, fill=0x33)
    out = bf16_host(d.forward(ws))
    go, claimed, done, err = _fused_words(ws)
    print(f"[gpu w4a8] T={T}: go={go:#x} items claimed={claimed} workgroups={done} err={err}", flush=True)
    assert go == 0 and err == 0 and done > 0 and claimed >= done
    assert (out == bf16_host(d0.forward())).all()
    # a smaller problem on the same (larger) workspace, then this one again
    inp2, d2 = sweep_case(max(1, T // 4))
    d2 = single_launch(inp2)
    n2 = tpg.moe_workspace_bytes(d2.p)
    o2 = torch.full((d2.cfg.T, d2.cfg.H), -1, dtype=torch.int16, device=DEV)
    tpg.moe_forward(d2.logits, d2.drop, d2.x, d2.x_scale, d2.weights, d2.p, o2, ws, n2)
    assert (bf16_host(o2) == bf16_host(d2.forward())).all()
    assert (bf16_host(d.forward(ws)) == out).all()
    assert _fused_words(ws)[0] == 0 and _fused_words(ws)[3] == 0


def test_forward_deterministic_and_workspace_reuse():
    _, d = sweep_case(128)
    ws = d.workspace(tpg.MOE_WS_FORWARD, fill=0x00)
    a = bf16_host(d.forward(ws))
    b = bf16_host(d.forward(ws))
    c = bf16_host(d.forward())
    assert (a == b).all() and (a == c).all()



def test_forward_at_the_gather_offset_limit():
    """T*H = 2^31 fp8 bytes of x: the forward gathers the rows and their scales with the separate
    permute kernel instead of inside GEMM1; sampled tokens against the oracle, every token row
    written, and bitwise the step-by-step entry points"""
    cfg = MoeConfig("w4_gather_limit", T=65536, H=32768, I=256, E=2, k=1, prec="w4a8", swiglu_clamp=10.0)
    print(f"[gpu w4a8] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    inp = generate(cfg, seed=7)
    d = DeviceProblem(inp)
    out_dev = d.forward()
    tokens = np.unique(np.concatenate([np.random.default_rng(7).integers(0, cfg.T, 14), [0, cfg.T - 1]]))
    ref = oracle.moe_forward(inp, tokens)
    out = bf16_host(out_dev)
    err = rel_err(bf16_f64(out[tokens]), ref)
    print(f"[gpu w4a8] {cfg.name}: forward on {tokens.size} tokens, max|err|/max|ref| = {err:.3e}", flush=True)
    assert err <= W4A8_BAR
    assert_all_rows_written(out_dev, cfg.T, float(np.abs(ref).max()), f"{cfg.name} forward out")
    del out_dev
    idx, w = d.route()
    offsets, row_src, slot_row, x_perm, x_perm_scale = d.permute(idx)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    del x_perm
    steps = bf16_host(d.combine(y, slot_row, w))
    assert (steps == out).all()


@pytest.mark.parametrize("prec", ["w4a8", "w4a8_mx"])
def test_forward_at_the_largest_hidden_size(prec):
    """H = 65536, the largest the boundary accepts: 256 K chunks in GEMM1 (the persistent form: sixteen tokens,
    so every tile holds one token block) and 512 n-tiles in GEMM2; every token against the oracle and every token row written"""
    cfg = MoeConfig(f"{prec}_max_h", T=16, H=65536, I=1024, E=4, k=2, prec=prec, swiglu_clamp=10.0)
    print(f"[gpu w4a8] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    inp = generate(cfg, seed=8)
    d = DeviceProblem(inp)
    out_dev = d.forward()
    ref = oracle.moe_forward(inp)
    err = rel_err(bf16_f64(bf16_host(out_dev)), ref)
    print(f"[gpu w4a8] {cfg.name}: forward, max|err|/max|ref| = {err:.3e}", flush=True)
    assert err <= W4A8_BAR
    assert_all_rows_written(out_dev, cfg.T, float(np.abs(ref).max()), f"{cfg.name} forward out")
