"""GPU parity: every entry point of the C ABI against the CPU oracle on the same
seeded inputs.

Bars: routing ids, permutation tables and offsets bit-exact; permuted rows
bit-exact copies; bf16 outputs max|err| / max|ref| <= 2e-2 against the fp64
oracle; routing weights within 2e-6 of the fp64 values.  Full-size workloads are
checked in full where the oracle is cheap (routing, tables, permutation) and on
sampled rows / tokens where it is not (expert FFN, forward); the sample always
holds the first and last row of every non-empty expert (every ragged tile tail)
and two whole 256-row m-tiles (an interior one of the largest expert, the first of
the median expert).  Every output buffer starts filled with 0xFFFF: at every size
each live row must have left that fill, with no magnitude far above the sampled
reference's, and rows past the live count must still hold it.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import token_permute_grouped_amd as tpg
from moe_synth import CONFIGS, MoeConfig, bf16_bits_from_f32, deinterleave_rows, generate
from tests._gpu import DEV, DeviceProblem, assert_all_rows_written, bf16_f64, bf16_host, rel_err, to_dev, \
    whole_tiles

pytestmark = pytest.mark.gpu

BF16_BAR = 2e-2
SMALL_CASES = {
    "tiny": CONFIGS["tiny"],
    "odd_T": MoeConfig("odd_T", T=3, H=128, I=128, E=8, k=2),
    "one_token": MoeConfig("one_token", T=1, H=256, I=384, E=4, k=4),
    "max_experts": MoeConfig("max_experts", T=300, H=128, I=128, E=256, k=32),
    "interleaved_drop": MoeConfig("interleaved_drop", T=200, H=256, I=256, E=16, k=4, glu_interleave=32,
                                  drop_p=0.1),
    "clamped": MoeConfig("clamped", T=150, H=384, I=256, E=8, k=3, swiglu_clamp=1.0),
    "ragged_tiles": MoeConfig("ragged_tiles", T=700, H=256, I=640, E=5, k=2),
    "wide_k": MoeConfig("wide_k", T=40, H=128, I=128, E=128, k=64),          # k above 32: 16 slots per lane
    "all_experts": MoeConfig("all_experts", T=8, H=128, I=128, E=256, k=256),  # k = E = 256: every expert, 8 rows each
}
FULL = ["mid", "skewed", "ep_share"]


@functools.lru_cache(maxsize=None)
def workload(name: str, seed: int = 0):
    cfg = SMALL_CASES.get(name) or CONFIGS[name]
    print(f"[gpu parity] generating {name} seed={seed} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}",
          flush=True)
    inp = generate(cfg, seed=seed)
    return inp, DeviceProblem(inp)


def _sample_rows(offsets: np.ndarray, extra: int, seed: int) -> np.ndarray:
    """first and last row of every non-empty expert plus `extra` random rows"""
    rows = []
    for e in range(offsets.size - 1):
        if offsets[e + 1] > offsets[e]:
            rows += [offsets[e], offsets[e + 1] - 1]
    R = int(offsets[-1])
    rows += list(np.random.default_rng(seed).integers(0, R, extra))
    return np.unique(np.array(rows, dtype=np.int64))


def _cases_all():
    return list(SMALL_CASES) + FULL


# ----------------------------------------------------------------------------- routing

@pytest.mark.parametrize("name", _cases_all())
def test_route_bit_exact(name):
    inp, d = workload(name)
    cfg = inp["cfg"]
    idx, w = d.route()
    ref_idx, ref_w = oracle.route(inp["logits"], cfg.k, inp.get("slot_drop"))
    assert (idx.cpu().numpy() == ref_idx).all()
    assert np.abs(w.cpu().numpy().astype(np.float64) - ref_w).max() <= 2e-6


def test_route_ties_and_equal_logits():
    cfg = MoeConfig("ties", T=256, H=128, I=128, E=64, k=8)
    rng = np.random.default_rng(1)
    lg = rng.integers(0, 4, size=(cfg.T, cfg.E)).astype(np.float32)
    lg[:8] = 0.5  # all equal
    inp = {"cfg": cfg, "logits": lg, "x": np.zeros((cfg.T, cfg.H), np.uint16),
           "w1": np.zeros((cfg.E, 2 * cfg.I, cfg.H), np.uint16), "w2": np.zeros((cfg.E, cfg.H, cfg.I), np.uint16)}
    d = DeviceProblem(inp)
    idx, w = d.route()
    ref_idx, ref_w = oracle.route(lg, cfg.k)
    assert (idx.cpu().numpy() == ref_idx).all()
    assert (idx.cpu().numpy()[:8] == np.arange(8)).all()
    assert (w.cpu().numpy()[:8] == np.float32(1 / 8)).all()


@pytest.mark.parametrize("E,k", [(200, 8), (256, 32), (3, 3), (130, 5), (64, 1), (256, 200), (48, 48)])
def test_route_exact_order_on_ties_signed_zeros_and_denormals(E, k):
    """selection is an exact comparison of the fp32 logits: ties (within and across lanes of a
    wave) go to the lower id, -0 equals +0, subnormals keep their order"""
    T = 120
    rng = np.random.default_rng(E * 100 + k)
    lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)          # many equal logits
    lg[1::4] *= np.float32(1e-40)                                        # subnormals, +-0
    sz = rng.random((T, E)) < 0.5
    lg[2::4] = np.where(sz[2::4], np.float32(-0.0), np.float32(0.0))     # only signed zeros
    lg[3::4] = np.where(sz[3::4], np.float32(-0.0), lg[3::4])            # zeros of both signs among ints
    cfg = MoeConfig("ties_zero_denorm", T=T, H=128, I=128, E=E, k=k)
    inp = {"cfg": cfg, "logits": lg, "x": np.zeros((T, cfg.H), np.uint16),
           "w1": np.zeros((E, 2 * cfg.I, cfg.H), np.uint16), "w2": np.zeros((E, cfg.H, cfg.I), np.uint16)}
    d = DeviceProblem(inp)
    idx, w = d.route()
    ref_idx, ref_w = oracle.route(lg, k)
    assert (idx.cpu().numpy() == ref_idx).all()
    assert np.abs(w.cpu().numpy().astype(np.float64) - ref_w).max() <= 2e-6
    assert (idx.cpu().numpy()[2::4] == np.arange(k)).all()               # all-zero rows: ids 0..k-1


# ----------------------------------------------------------------------------- permutation

@pytest.mark.parametrize("name", _cases_all())
def test_permute_tables_and_rows_bit_exact(name):
    inp, d = workload(name)
    cfg = inp["cfg"]
    idx, _ = d.route()
    offsets, row_src, slot_row, x_perm, _ = d.permute(idx)
    torch.cuda.synchronize()
    _, ref_off, ref_rs, ref_sr = oracle.tables(idx.cpu().numpy(), cfg.E)
    assert (offsets.cpu().numpy() == ref_off).all()
    assert (row_src.cpu().numpy() == ref_rs).all()
    assert (slot_row.cpu().numpy() == ref_sr).all()
    R = int(ref_off[-1])
    xp = x_perm.cpu().numpy().view(np.uint16)
    assert (xp[:R] == inp["x"][ref_rs[:R] // cfg.k]).all()   # pure copy of each token row
    assert (xp[R:] == 0xFFFF).all()                          # canary rows past R untouched


# ----------------------------------------------------------------------------- combine

# expert ids chosen directly (no routing) around the one-workgroup tables kernel's bound of 2048
# slots: exactly 2048 and 2049 slots, every slot dropped, one hot expert, one expert, one slot
TABLE_CASES = [
    ("s2048_drops", 2048, 1, 64, "random"), ("s2049", 2049, 1, 64, "random"), ("s2048_k8", 256, 8, 256, "random"),
    ("s1024_all_dropped", 512, 2, 16, "dropped"), ("s2048_one_hot", 1024, 2, 256, "hot"),
    ("s1500_one_expert", 1500, 1, 1, "random"), ("s1", 1, 1, 4, "random"), ("s4100", 2050, 2, 33, "random"),
]


@pytest.mark.parametrize("case", TABLE_CASES, ids=[c[0] for c in TABLE_CASES])
def test_tables_bit_exact_at_the_one_workgroup_bound(case):
    name, T, k, E, mode = case
    print(f"[gpu parity] tables {name}: T={T} k={k} E={E} {mode}", flush=True)
    rng = np.random.default_rng(T * 31 + k * 7 + E)
    if mode == "dropped":
        idx = np.full((T, k), -1, np.int32)
    elif mode == "hot":
        idx = np.where(rng.random((T, k)) < 0.9, 5, rng.integers(0, E, (T, k))).astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
        idx[rng.random((T, k)) < 0.1] = -1  # dropped slots
    cfg = MoeConfig(name, T=T, H=128, I=128, E=E, k=k)
    inp = {"cfg": cfg, "logits": np.zeros((T, E), np.float32), "x": rng.integers(0, 1 << 16, (T, 128), dtype=np.uint16),
           "w1": np.zeros((E, 256, 128), np.uint16), "w2": np.zeros((E, 128, 128), np.uint16)}
    d = DeviceProblem(inp)
    offsets, row_src, slot_row, x_perm, _ = d.permute(to_dev(idx))
    torch.cuda.synchronize()
    _, ref_off, ref_rs, ref_sr = oracle.tables(idx, E)
    assert (offsets.cpu().numpy() == ref_off).all()
    assert (row_src.cpu().numpy() == ref_rs).all()
    assert (slot_row.cpu().numpy() == ref_sr).all()
    R = int(ref_off[-1])
    assert (x_perm.cpu().numpy().view(np.uint16)[:R] == inp["x"][ref_rs[:R] // k]).all()


@pytest.mark.parametrize("name", ["tiny", "interleaved_drop", "max_experts", "mid"])
def test_combine_matches_oracle(name):
    inp, d = workload(name)
    cfg = inp["cfg"]
    idx, w = d.route()
    _, _, slot_row, _, _ = d.permute(idx)
    rng = np.random.default_rng(7)
    y_bits = bf16_bits_from_f32(rng.standard_normal((d.S, cfg.H)).astype(np.float32))
    out = d.combine(to_dev(y_bits), slot_row, w)
    got = bf16_f64(bf16_host(out))
    ref = oracle.combine_bf16(y_bits, slot_row.cpu().numpy(), w.cpu().numpy(), cfg.T, cfg.k)
    # fp32 accumulation then one bf16 rounding: within one bf16 ulp of the fp64 sum
    assert (np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-6).all()


@pytest.mark.parametrize("name", ["tiny", "interleaved_drop", "max_experts"])
def test_identity_experts_return_x(name):
    """permute, identity experts, combine with weights renormalised over valid slots: out == x bitwise"""
    inp, d = workload(name)
    cfg = inp["cfg"]
    idx, w = d.route()
    offsets, row_src, slot_row, x_perm, _ = d.permute(idx)
    iv = idx.cpu().numpy()
    wv = np.where(iv >= 0, w.cpu().numpy(), 0).astype(np.float64)
    keep = wv.sum(axis=1) > 0
    wv[keep] /= wv[keep].sum(axis=1, keepdims=True)
    out = d.combine(x_perm, slot_row, to_dev(wv.astype(np.float32)))
    got = bf16_host(out)
    assert (got[keep] == inp["x"][keep]).all()
    assert (got[~keep] == 0).all()


# ----------------------------------------------------------------------------- expert FFN

@pytest.mark.parametrize("name", list(SMALL_CASES) + FULL)
def test_grouped_ffn_rows(name):
    inp, d = workload(name)
    cfg = inp["cfg"]
    idx, _ = d.route()
    offsets, row_src, slot_row, x_perm, x_perm_scale = d.permute(idx)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    torch.cuda.synchronize()
    off = offsets.cpu().numpy()
    rs = row_src.cpu().numpy()
    R = int(off[-1])
    small = name in SMALL_CASES
    rows = np.arange(R) if small else np.union1d(_sample_rows(off, extra=32, seed=1), whole_tiles(off, 256))
    expert = np.searchsorted(off, rows, side="right") - 1
    ref = oracle.ffn_rows(inp, rs[rows] // cfg.k, expert)
    got = bf16_f64(bf16_host(y)[rows])
    err = rel_err(got, ref)
    print(f"[gpu parity] {name}: grouped FFN on {rows.size} rows, max|err|/max|ref| = {err:.3e}")
    assert err <= BF16_BAR
    assert_all_rows_written(y, R, float(np.abs(ref).max()), f"{name} y_perm")
    assert (bf16_host(y)[R:] == 0xFFFF).all()   # rows past R not written


def test_interleave_32_equals_plain_layout():
    inp, d = workload("interleaved_drop")
    cfg = inp["cfg"]
    plain_cfg = MoeConfig("plain", T=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, k=cfg.k, drop_p=cfg.drop_p)
    plain = dict(inp, cfg=plain_cfg, w1=deinterleave_rows(inp["w1"], cfg.I, 32))
    d2 = DeviceProblem(plain)
    a = bf16_host(d.forward())
    b = bf16_host(d2.forward())
    assert (a == b).all()   # same products in the same order: bitwise equal


# ----------------------------------------------------------------------------- whole forward

@pytest.mark.parametrize("name", list(SMALL_CASES) + FULL)
def test_forward_matches_oracle(name):
    inp, d = workload(name)
    cfg = inp["cfg"]
    out = bf16_host(d.forward())
    if name in SMALL_CASES:
        tokens = np.arange(cfg.T)
    else:
        tokens = np.unique(np.concatenate([np.random.default_rng(3).integers(0, cfg.T, 24), [0, cfg.T - 1]]))
    ref = oracle.moe_forward(inp, tokens)
    err = rel_err(bf16_f64(out[tokens]), ref)
    print(f"[gpu parity] {name}: forward on {tokens.size} tokens, max|err|/max|ref| = {err:.3e}")
    assert err <= BF16_BAR
    assert_all_rows_written(to_dev(out), cfg.T, float(np.abs(ref).max()), f"{name} forward out")


@pytest.mark.parametrize("cfg", [
    MoeConfig("front_tiny", T=64, H=128, I=256, E=8, k=2),
    MoeConfig("front_drop", T=30, H=256, I=256, E=16, k=4, glu_interleave=32, drop_p=0.1),
    MoeConfig("front_e256", T=32, H=128, I=128, E=256, k=32),             # exactly 1024 slots
    MoeConfig("front_one", T=1, H=256, I=384, E=4, k=4),
    MoeConfig("front_t128", T=128, H=256, I=256, E=32, k=8, drop_p=0.05),   # 1024 slots, two routing passes
    MoeConfig("front_t256", T=256, H=128, I=128, E=64, k=4),             # 256 tokens: four passes
    MoeConfig("front_t100_odd", T=100, H=128, I=256, E=12, k=3),         # last pass partly empty
    MoeConfig("front_wide_k", T=8, H=128, I=128, E=256, k=100, drop_p=0.1),  # k above 32 in the front end
    # just past the bound (1024 slots): the separate launches, two table chunks
    MoeConfig("front_1025", T=205, H=128, I=128, E=16, k=5),              # one slot in the second chunk
    MoeConfig("front_1500_drop", T=250, H=128, I=256, E=12, k=6, drop_p=0.1),
    MoeConfig("front_2048", T=256, H=128, I=128, E=32, k=8),
    MoeConfig("front_k16", T=128, H=256, I=128, E=64, k=16, glu_interleave=32),
    MoeConfig("front_2050", T=205, H=128, I=128, E=16, k=10),
    MoeConfig("front_w4_2048", T=256, H=512, I=512, E=32, k=8, prec="w4a8", swiglu_clamp=10.0, drop_p=0.02),
    MoeConfig("front_mx_1536", T=192, H=512, I=512, E=16, k=8, prec="w4a8_mx"),
], ids=lambda c: c.name)
def test_forward_small_front_end_matches_separate_steps(cfg):
    """up to 1024 slots and 256 tokens the forward routes, builds the tables and the tile
    list in one launch; it must give exactly what the separate entry points give"""
    inp = generate(cfg, seed=2)
    d = DeviceProblem(inp)
    fused = bf16_host(d.forward())
    idx, w = d.route()
    offsets, row_src, slot_row, x_perm, x_perm_scale = d.permute(idx)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    steps = bf16_host(d.combine(y, slot_row, w))
    assert (fused == steps).all()


@pytest.mark.parametrize("name", ["ragged_tiles", "interleaved_drop", "clamped", "max_experts"] + FULL)
def test_forward_gather_in_gemm1_equals_separate_steps(name):
    """the bf16 forward reads x through row_src inside GEMM1 instead of gathering x_perm first;
    its output must be bitwise what route + permute + grouped FFN + combine give"""
    inp, d = workload(name)
    fused = bf16_host(d.forward())
    idx, w = d.route()
    offsets, row_src, slot_row, x_perm, x_perm_scale = d.permute(idx, canary=False)
    y = d.grouped_ffn(x_perm, x_perm_scale, offsets)
    steps = bf16_host(d.combine(y, slot_row, w))
    del y, x_perm
    n_diff = int((fused != steps).sum())
    print(f"[gpu parity] {name}: fused-gather forward vs separate steps, {n_diff} differing elements")
    assert n_diff == 0


@pytest.mark.parametrize("name", ["tiny", "skewed"])
def test_forward_is_deterministic(name):
    _, d = workload(name)
    ws = d.workspace(tpg.MOE_WS_FORWARD)
    a = bf16_host(d.forward(ws))
    b = bf16_host(d.forward(ws))
    assert (a == b).all()


def test_workspace_reuse_across_routings():
    """a workspace left by one routing must not leak into the next call (the hot-expert cleanup lesson)"""
    _, da = workload("ragged_tiles", 0)
    _, db = workload("ragged_tiles", 1)
    ws = da.workspace(tpg.MOE_WS_FORWARD, fill=0x00)
    da.forward(ws)
    b_reused = bf16_host(db.forward(ws))
    b_fresh = bf16_host(db.forward())
    assert (b_reused == b_fresh).all()


def test_empty_experts():
    cfg = MoeConfig("empty", T=128, H=128, I=256, E=16, k=2)
    inp = generate(cfg, seed=5)
    inp["logits"][:, [0, 5, 6, 15]] -= 1000.0   # experts 0, 5, 6 and 15 are never chosen
    d = DeviceProblem(inp)
    idx, _ = d.route()
    offsets, *_ = d.permute(idx)
    off = offsets.cpu().numpy()
    assert all(off[e + 1] == off[e] for e in (0, 5, 6, 15))
    out = bf16_host(d.forward())
    err = rel_err(bf16_f64(out), oracle.moe_forward(inp))
    assert err <= BF16_BAR


def test_zero_tokens_is_a_no_op():
    p = tpg.make_problem(0, 128, 128, 8, 2)
    out = torch.full((4,), 7, dtype=torch.int16, device=DEV)
    w = tpg.make_weights(out, out)
    tpg.moe_forward(None, None, None, None, w, p, out, None)
    tpg.moe_unpermute_combine(None, None, None, p, out)
    torch.cuda.synchronize()
    assert (out.cpu() == 7).all()


def test_forward_at_the_gather_offset_limit():
    """T*H*2 = 2^31 bytes of x: the rows no longer fit one buffer descriptor's 31-bit offsets, so the
    forward gathers them with the separate permute kernel instead of inside GEMM1; sampled tokens
    against the oracle, every token row written, and bitwise the step-by-step entry points"""
    cfg = MoeConfig("gather_limit", T=32768, H=32768, I=128, E=2, k=1)
    print(f"[gpu parity] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    inp = generate(cfg, seed=7)
    d = DeviceProblem(inp)
    out_dev = d.forward()
    tokens = np.unique(np.concatenate([np.random.default_rng(7).integers(0, cfg.T, 14), [0, cfg.T - 1]]))
    ref = oracle.moe_forward(inp, tokens)
    out = bf16_host(out_dev)
    err = rel_err(bf16_f64(out[tokens]), ref)
    print(f"[gpu parity] {cfg.name}: forward on {tokens.size} tokens, max|err|/max|ref| = {err:.3e}", flush=True)
    assert err <= BF16_BAR
    assert_all_rows_written(out_dev, cfg.T, float(np.abs(ref).max()), f"{cfg.name} forward out")
    del out_dev
    idx, w = d.route()
    offsets, row_src, slot_row, x_perm, _ = d.permute(idx)
    y = d.grouped_ffn(x_perm, None, offsets)
    del x_perm
    steps = bf16_host(d.combine(y, slot_row, w))
    assert (steps == out).all()


def test_forward_at_the_largest_hidden_size():
    """H = 65536, the largest the boundary accepts: 1024 K stages in GEMM1 and 256 n-tiles in GEMM2;
    every token against the oracle and every token row written"""
    cfg = MoeConfig("max_h", T=64, H=65536, I=1024, E=2, k=2)
    print(f"[gpu parity] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}", flush=True)
    inp = generate(cfg, seed=8)
    d = DeviceProblem(inp)
    out_dev = d.forward()
    ref = oracle.moe_forward(inp)
    err = rel_err(bf16_f64(bf16_host(out_dev)), ref)
    print(f"[gpu parity] {cfg.name}: forward, max|err|/max|ref| = {err:.3e}", flush=True)
    assert err <= BF16_BAR
    assert_all_rows_written(out_dev, cfg.T, float(np.abs(ref).max()), f"{cfg.name} forward out")
