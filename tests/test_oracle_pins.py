"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to something independent of it: a value the
source pages state, a library routine (torch's float8_e4m3fn cast, numpy matmul,
scipy's softmax and expit, Python's stable sort), brute force over tiny inputs,
a closed form, or an invariant of the method.  The inputs are random and
asymmetric, so a dropped term, a wrong sign or index, or a transposed operand in
the oracle fails at least one of them.
"""
import dataclasses
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from moe_synth import CONFIGS, MoeConfig, bf16_bits_from_f32, bf16_bits_to_f32, deinterleave_rows, generate
from moe_synth.gen import E2M1_VALUES, _interleave_perm


# ----------------------------------------------------------------------------- number formats

def _torch_e4m3(code):
    t = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn)
    return float(t.to(torch.float64)[0])


def test_e4m3_decode_all_codes_match_torch():
    for c in range(256):
        want = _torch_e4m3(c)
        got = oracle.e4m3_value(c)
        if np.isnan(want):
            assert np.isnan(got), c
        else:
            assert got == want, (c, got, want)


def test_e4m3_max_is_448():
    # FlashInfer #6517 (weight preparation): NVFP4 block scales must satisfy 6*scale <= 448,
    # i.e. 448 is the largest finite E4M3 value and 6 the largest E2M1 value.
    finite = [oracle.e4m3_value(c) for c in range(256) if not np.isnan(oracle.e4m3_value(c))]
    assert max(finite) == 448.0 and min(finite) == -448.0
    assert max(oracle.e2m1_value(c) for c in range(16)) == 6.0


def test_e2m1_decode_matches_ocp_value_set():
    # OCP MX specification, FP4 E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
    for c in range(16):
        mag = E2M1_VALUES[c & 7]
        assert oracle.e2m1_value(c) == (-mag if c & 8 else mag)


def test_e4m3_encode_matches_torch_cast_on_every_midpoint():
    vals = sorted({_torch_e4m3(c) for c in range(127)})  # non-negative finite values
    probes = []
    for a, b in zip(vals[:-1], vals[1:]):
        m = (a + b) / 2
        probes += [a, b, m, np.nextafter(m, 0, dtype=np.float64), np.nextafter(m, 1e9, dtype=np.float64)]
    probes = np.array(probes, dtype=np.float32)  # fp32 inputs, as the kernel sees them
    rng = np.random.default_rng(5)
    probes = np.concatenate([probes, rng.standard_normal(20000).astype(np.float32) * 30,
                             rng.standard_normal(5000).astype(np.float32) * 1e-2, [0.0, -0.0, 447.9, 448.0]])
    probes = np.concatenate([probes, -probes]).astype(np.float32)
    want = torch.from_numpy(probes).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in probes], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(probes[i], got[i], want[i]) for i in bad[:10]]


def test_e4m3_encode_nan_is_the_nan_code_with_its_sign():
    for v, code in [(float("nan"), 0x7F), (-float("nan"), 0xFF)]:
        want = int(torch.tensor([v]).to(torch.float8_e4m3fn).view(torch.uint8)[0])
        assert oracle.e4m3_encode(v) == want == code


def test_e4m3_encode_saturates():
    # torch's cast overflows to NaN beyond 464; the reading used here (and on the GPU) saturates.
    for v in [448.0, 449.0, 464.0, 465.0, 1e6, 1e30]:
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE


def test_fp4_to_fp8_dequant_table_matches_torch():
    tab = oracle.fp4_to_fp8_table()
    for c in range(16):
        for s in range(256):
            sv = _torch_e4m3(s)
            if np.isnan(sv):    # outside the defined domain: the NaN code carrying the product's sign
                neg = bool(c & 8) != bool(s & 0x80)
                nan = torch.tensor([-float("nan") if neg else float("nan")]).to(torch.float8_e4m3fn)
                assert tab[c, s] == int(nan.view(torch.uint8)[0]), (c, s)
                continue
            prod = np.float32(E2M1_VALUES[c & 7] * (-1 if c & 8 else 1) * sv)  # exact: <= 5 significant bits
            want = torch.tensor([np.clip(prod, -448, 448)], dtype=torch.float32).to(torch.float8_e4m3fn)
            assert tab[c, s] == int(want.view(torch.uint8)[0]), (c, s)


# ----------------------------------------------------------------------------- routing

def _route_brute(lg, k):
    """k-subset of maximum total logit (unique for distinct logits), ordered by (-logit, id)."""
    E = lg.size
    best = max(itertools.combinations(range(E), k), key=lambda sub: sum(float(lg[e]) for e in sub))
    return sorted(best, key=lambda e: (-float(lg[e]), e))


@pytest.mark.parametrize("E,k", [(4, 1), (6, 2), (8, 3), (9, 4), (7, 7)])
def test_route_brute_force(E, k):
    rng = np.random.default_rng(E * 10 + k)
    lg = rng.standard_normal((40, E)).astype(np.float32)
    idx, w = oracle.route(lg, k)
    for t in range(lg.shape[0]):
        assert list(idx[t]) == _route_brute(lg[t], k)
        p = scipy.special.softmax(lg[t].astype(np.float64))
        sel = p[idx[t]]
        np.testing.assert_allclose(w[t], sel / sel.sum(), rtol=1e-13)
        assert abs(w[t].sum() - 1) < 1e-14
        assert np.all(np.diff(w[t]) <= 0)


def test_route_ties_go_to_lower_id():
    rng = np.random.default_rng(3)
    lg = rng.integers(0, 3, size=(200, 8)).astype(np.float32)  # many ties
    idx, _ = oracle.route(lg, 3)
    for t in range(lg.shape[0]):
        assert list(idx[t]) == sorted(range(8), key=lambda e: (-lg[t, e], e))[:3]


def test_route_all_equal_logits():
    lg = np.full((5, 16), 0.25, np.float32)
    idx, w = oracle.route(lg, 4)
    assert (idx == np.arange(4)).all()
    assert (w == 0.25).all()


def test_route_single_expert_weight_is_exactly_one():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((50, 6)).astype(np.float32)
    idx, w = oracle.route(lg, 1)
    assert (w == 1.0).all()
    assert (idx[:, 0] == np.argmax(lg, axis=1)).all()


def test_route_slot_drop_masks_without_renormalising():
    rng = np.random.default_rng(12)
    lg = rng.standard_normal((30, 8)).astype(np.float32)
    drop = (rng.random((30, 3)) < 0.4).astype(np.uint8)
    idx0, w0 = oracle.route(lg, 3)
    idx1, w1 = oracle.route(lg, 3, drop)
    assert (idx1 == np.where(drop == 1, -1, idx0)).all()
    assert (w1 == w0).all()


# ----------------------------------------------------------------------------- tables

def _tables_brute(idx, E):
    S = idx.size
    flat = idx.reshape(-1)
    order = sorted((s for s in range(S) if flat[s] >= 0), key=lambda s: (flat[s], s))  # stable by (expert, slot)
    counts = np.array([(flat == e).sum() for e in range(E)], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_src = np.full(S, -1, np.int32)
    row_src[: len(order)] = order
    slot_row = np.full(S, -1, np.int32)
    for r, s in enumerate(order):
        slot_row[s] = r
    return counts, offsets, row_src, slot_row


@pytest.mark.parametrize("T,E,k,p_drop", [(1, 4, 2, 0.0), (37, 8, 2, 0.0), (50, 16, 4, 0.3), (64, 3, 3, 0.0)])
def test_tables_brute_force(T, E, k, p_drop):
    rng = np.random.default_rng(T + E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    drop = (rng.random((T, k)) < p_drop).astype(np.uint8) if p_drop else None
    idx, _ = oracle.route(lg, k, drop)
    got = oracle.tables(idx, E)
    want = _tables_brute(idx, E)
    for g, w in zip(got, want):
        assert (g == w).all()


def test_tables_invariants_skewed_workload():
    inp = generate(CONFIGS["skewed"], seed=3, weights=False)  # seed 3 leaves one expert empty
    cfg = inp["cfg"]
    idx, _ = oracle.route(inp["logits"], cfg.k)
    counts, offsets, row_src, slot_row = oracle.tables(idx, cfg.E)
    assert counts.sum() == cfg.T * cfg.k                    # expert counts sum to T*k
    assert (np.diff(offsets) == counts).all() and offsets[0] == 0
    assert (counts == 0).any()                               # Zipf skew: empty experts ...
    assert counts.max() > 100 * np.median(counts)             # ... and very ragged groups
    R = offsets[-1]
    assert (slot_row[row_src[:R]] == np.arange(R)).all()     # row_src o slot_row = id
    assert np.unique(row_src[:R]).size == R
    flat = idx.reshape(-1)
    for e in range(cfg.E):                                   # segment e holds expert e's slots, ascending
        seg = row_src[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def test_tables_with_dropped_slots():
    inp = generate(CONFIGS["ep_share"], seed=1, T=2048, weights=False)
    cfg = inp["cfg"]
    idx, _ = oracle.route(inp["logits"], cfg.k, inp["slot_drop"])
    counts, offsets, row_src, slot_row = oracle.tables(idx, cfg.E)
    n_drop = int(inp["slot_drop"].sum())
    assert 0.07 < n_drop / idx.size < 0.13
    assert counts.sum() == idx.size - n_drop
    assert ((slot_row == -1) == (idx.reshape(-1) == -1)).all()
    assert (row_src[offsets[-1]:] == -1).all()


# ----------------------------------------------------------------------------- permute / combine

@pytest.mark.parametrize("name,T", [("tiny", 64), ("ep_share", 256)])
def test_permute_then_combine_with_identity_experts_returns_x(name, T):
    cfg = CONFIGS[name]
    small = MoeConfig("t", T=T, H=256, I=128, E=cfg.E, k=cfg.k, drop_p=cfg.drop_p)
    inp = generate(small, seed=2, weights=False)
    idx, w = oracle.route(inp["logits"], small.k, inp["slot_drop"])
    valid = idx >= 0
    keep = valid.any(axis=1)
    wv = np.where(valid, w, 0.0)
    wv[keep] /= wv[keep].sum(axis=1, keepdims=True)            # renormalise over valid slots
    counts, offsets, row_src, slot_row = oracle.tables(idx, small.E)
    R = int(offsets[-1])
    x_perm = oracle.permute_rows(inp["x"], row_src, R, small.k)
    xs = inp["x"][row_src[:R] // small.k]
    assert (x_perm == xs).all()                                 # pure row copy
    out = oracle.combine_bf16(x_perm, slot_row, wv.astype(np.float32), small.T, small.k)
    got = bf16_bits_from_f32(out.astype(np.float32))
    assert (got[keep] == inp["x"][keep]).all()
    assert (out[~keep] == 0).all()


def _fingerprint_combine_case(seed, T=48, k=4, E=8, H=24, p_drop=0.2):
    """Routing with dropped slots, tables from Python's stable sort, distinct random integer rows
    per slot (|y| < 128, exact in bf16), and weights (1 + m/8) 2^-12j per slot j (m < 8): term j of
    a token's sum is an integer below 2^11 in magnitude times 2^(-3-12j), so the terms sit in
    disjoint 12-bit bands, the fp64 sum is exact (47 bits for k = 4) and records which row was
    paired with which slot's weight; any other pairing changes it."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[rng.random((T, k)) < p_drop] = -1
    idx[0] = -1                                              # a token with every slot dropped
    _, _, row_src, slot_row = _tables_brute(idx, E)
    R = int((idx >= 0).sum())
    y = rng.integers(-127, 128, (max(R, 1), H)).astype(np.float32)
    y_bits = bf16_bits_from_f32(y)
    assert (bf16_bits_to_f32(y_bits) == y).all()
    m = rng.integers(0, 8, (T, k))
    w = (np.ldexp(1.0 + m / 8.0, -12 * np.arange(k)[None, :])).astype(np.float32)
    return idx, row_src, slot_row, y_bits, y.astype(np.float64), w


def _combine_by_definition(idx, row_src, y, w):
    """out[t] = sum over the token's valid slots j of w[t, j] times the row that holds slot t*k+j,
    in Python fractions (exact); the row of a slot is found by scanning row_src."""
    from fractions import Fraction
    T, k = idx.shape
    where = {int(s): r for r, s in enumerate(row_src) if s >= 0}
    out = np.zeros((T, y.shape[1]))
    for t in range(T):
        for c in range(y.shape[1]):
            acc = Fraction(0)
            for j in range(k):
                if idx[t, j] >= 0:
                    acc += Fraction(float(w[t, j])) * Fraction(float(y[where[t * k + j], c]))
            out[t, c] = float(acc)                           # exact: the bands never overlap
    return out


def test_combine_pairs_each_weight_with_its_own_slot_row():
    idx, row_src, slot_row, y_bits, y, w = _fingerprint_combine_case(seed=31)
    T, k = idx.shape
    want = _combine_by_definition(idx, row_src, y, w)
    got = oracle.combine_bf16(y_bits, slot_row, w, T, k)
    assert np.array_equal(got, want)
    assert (got[0] == 0).all()                               # all slots dropped: 0
    # the same pin rejects the outputs of a combine that mispairs: weights of slots 0 and 1 swapped
    # within each token, or each slot read from its neighbour's row
    w_swapped = w.copy()
    w_swapped[:, [0, 1]] = w[:, [1, 0]]
    assert not np.array_equal(oracle.combine_bf16(y_bits, slot_row, w_swapped, T, k), want)
    sr = slot_row.reshape(T, k)
    sr_rot = np.where((sr >= 0).all(axis=1, keepdims=True), np.roll(sr, 1, axis=1), sr).reshape(-1)
    assert (sr_rot != slot_row).any()
    assert not np.array_equal(oracle.combine_bf16(y_bits, sr_rot, w, T, k), want)


def test_combine_equals_a_scatter_matrix_product():
    """General values: out = C Y with C[t, r] = w[t, j] where row r holds slot (t, j) (numpy fp64
    matmul on the brute-force tables)"""
    rng = np.random.default_rng(32)
    T, k, E, H = 64, 6, 16, 40
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[rng.random((T, k)) < 0.15] = -1
    _, _, row_src, slot_row = _tables_brute(idx, E)
    R = int((idx >= 0).sum())
    y_bits = bf16_bits_from_f32(rng.standard_normal((R, H)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32)
    C = np.zeros((T, R))
    for r in range(R):
        s = int(row_src[r])
        C[s // k, r] = w[s // k, s % k]
    want = C @ bf16_bits_to_f32(y_bits).astype(np.float64)
    got = oracle.combine_bf16(y_bits, slot_row, w, T, k)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------- expert FFN

def _dense_mlp(x, w1_logical, w2, I, clamp=0.0):
    """numpy fp64: silu(x Wg^T) * (x Wu^T) W2^T, optional clamp on both GLU inputs"""
    g = x @ w1_logical[:I].T
    u = x @ w1_logical[I:].T
    if clamp:
        g, u = np.clip(g, -clamp, clamp), np.clip(u, -clamp, clamp)
    return (g * scipy.special.expit(g) * u) @ w2.T


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("il", [0, 32])
def test_top1_equals_dense_swiglu_mlp(il):
    cfg = MoeConfig("t", T=48, H=128, I=192, E=4, k=1, glu_interleave=il)
    inp = generate(cfg, seed=4)
    out = oracle.moe_forward(inp)
    e = np.argmax(inp["logits"], axis=1)
    x = _f64(inp["x"])
    for t in range(cfg.T):
        w1l = deinterleave_rows(_f64(inp["w1"][e[t]]), cfg.I, il)
        want = _dense_mlp(x[t:t + 1], w1l, _f64(inp["w2"][e[t]]), cfg.I)[0]
        np.testing.assert_allclose(out[t], want, rtol=1e-11, atol=1e-12)


def test_topk_forward_equals_weighted_dense_mlps():
    cfg = CONFIGS["tiny"]
    inp = generate(cfg, seed=1)
    out = oracle.moe_forward(inp)
    x = _f64(inp["x"])
    lg = inp["logits"].astype(np.float64)
    for t in range(cfg.T):
        p = scipy.special.softmax(lg[t])
        sel = np.argsort(-p, kind="stable")[: cfg.k]
        w = p[sel] / p[sel].sum()
        want = sum(w[j] * _dense_mlp(x[t:t + 1], _f64(inp["w1"][e]), _f64(inp["w2"][e]), cfg.I)[0]
                   for j, e in enumerate(sel))
        np.testing.assert_allclose(out[t], want, rtol=1e-10, atol=1e-12)


def test_dropped_slots_are_skipped():
    cfg = MoeConfig("t", T=32, H=128, I=128, E=8, k=3, drop_p=0.3)
    inp = generate(cfg, seed=6)
    out = oracle.moe_forward(inp)
    idx, w = oracle.route(inp["logits"], cfg.k, inp["slot_drop"])
    x = _f64(inp["x"])
    for t in range(cfg.T):
        want = np.zeros(cfg.H)
        for j in range(cfg.k):
            if idx[t, j] >= 0:
                e = idx[t, j]
                want += w[t, j] * _dense_mlp(x[t:t + 1], _f64(inp["w1"][e]), _f64(inp["w2"][e]), cfg.I)[0]
        np.testing.assert_allclose(out[t], want, rtol=1e-10, atol=1e-12)
    all_dropped = (idx < 0).all(axis=1)
    assert (out[all_dropped] == 0).all()


def test_ffn_closed_forms():
    cfg = MoeConfig("t", T=16, H=128, I=128, E=2, k=2)
    inp = generate(cfg, seed=7)
    tok = np.arange(16, dtype=np.int32)
    ex = (tok % 2).astype(np.int32)
    # W2 = 0  =>  y = 0
    z = dict(inp, w2=np.zeros_like(inp["w2"]))
    assert (oracle.ffn_rows(z, tok, ex) == 0).all()
    # x = 0  =>  y = 0
    z = dict(inp, x=np.zeros_like(inp["x"]))
    assert (oracle.ffn_rows(z, tok, ex) == 0).all()
    # one-hot W1 rows and identity W2: gate n reads x[a_n], up n reads x[b_n]  =>  y[n] = silu(x[a_n]) x[b_n]
    rng = np.random.default_rng(8)
    a, b = rng.integers(0, cfg.H, cfg.I), rng.integers(0, cfg.H, cfg.I)
    one = np.uint16(0x3F80)
    w1 = np.zeros_like(inp["w1"])
    w1[:, np.arange(cfg.I), a] = one
    w1[:, cfg.I + np.arange(cfg.I), b] = one
    w2 = np.zeros_like(inp["w2"])
    w2[:, np.arange(cfg.H), np.arange(cfg.H)] = one          # H == I here
    y = oracle.ffn_rows(dict(inp, w1=w1, w2=w2), tok, ex)
    x = _f64(inp["x"])
    want = x[:, a] * scipy.special.expit(x[:, a]) * x[:, b]
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=0)


def test_clamp_limits_both_glu_inputs():
    cfg = MoeConfig("t", T=8, H=128, I=128, E=1, k=1, swiglu_clamp=10.0)
    inp = generate(cfg, seed=9)
    inp["x"] = bf16_bits_from_f32(bf16_bits_to_f32(inp["x"]) * 64)  # drive |g|,|u| well past 10
    tok = np.arange(8, dtype=np.int32)
    ex = np.zeros(8, np.int32)
    y = oracle.ffn_rows(inp, tok, ex)
    want = _dense_mlp(_f64(inp["x"]), _f64(inp["w1"][0]), _f64(inp["w2"][0]), cfg.I, clamp=10.0)
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-12)
    unclamped = _dense_mlp(_f64(inp["x"]), _f64(inp["w1"][0]), _f64(inp["w2"][0]), cfg.I)
    assert np.abs(unclamped - want).max() > 1.0


def test_interleave_is_a_pure_reindexing():
    cfg = MoeConfig("t", T=24, H=128, I=256, E=3, k=2, glu_interleave=32)
    inp = generate(cfg, seed=10)
    plain = dict(inp, cfg=MoeConfig("t", T=24, H=128, I=256, E=3, k=2),
                 w1=deinterleave_rows(inp["w1"], cfg.I, 32))
    assert (oracle.moe_forward(inp) == oracle.moe_forward(plain)).all()   # bitwise


# ----------------------------------------------------------------------------- W4A8 expert FFN

def _torch_fp8_round(v32):
    t = torch.from_numpy(np.clip(v32, -448, 448).astype(np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _dequant_nvfp4(packed, bscale, gscale):
    codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[0], -1)
    mag = E2M1_VALUES[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    sc = torch.from_numpy(np.repeat(bscale, 16, axis=1)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return _torch_fp8_round((mag * sc).astype(np.float32)) * np.float64(gscale)


def test_w4a8_ffn_equals_dense_computation_on_dequantised_operands():
    cfg = MoeConfig("t", T=6, H=256, I=256, E=3, k=2, prec="w4a8", swiglu_clamp=10.0)
    inp = generate(cfg, seed=13)
    tok = np.array([0, 1, 2, 3, 4, 5, 0, 3], np.int32)
    ex = np.array([0, 1, 2, 0, 1, 2, 2, 1], np.int32)
    y = oracle.ffn_rows(inp, tok, ex)
    xq = torch.from_numpy(inp["x"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xd = xq * np.repeat(inp["x_scale"].astype(np.float64), 128, axis=1)
    for i, (t, e) in enumerate(zip(tok, ex)):
        w1 = _dequant_nvfp4(inp["w1"][e], inp["w1_bscale"][e], inp["w1_gscale"][e])
        w2 = _dequant_nvfp4(inp["w2"][e], inp["w2_bscale"][e], inp["w2_gscale"][e])
        g = np.clip(xd[t] @ w1[: cfg.I].T, -10, 10)
        u = np.clip(xd[t] @ w1[cfg.I:].T, -10, 10)
        h = (g * scipy.special.expit(g) * u).astype(np.float32).reshape(-1, 128)
        s = (np.abs(h).max(axis=1) / np.float32(448)).astype(np.float32)
        s[s == 0] = 1
        hq = _torch_fp8_round((h / s[:, None]).astype(np.float32)) * s[:, None].astype(np.float64)
        want = hq.reshape(-1) @ w2.T
        np.testing.assert_allclose(y[i], want, rtol=1e-9, atol=1e-12)


def test_w4a8_generator_respects_the_decoder_range():
    # FlashInfer #6517: NVFP4 block scales must satisfy 6 * scale <= 448.
    cfg = MoeConfig("t", T=4, H=256, I=128, E=2, k=1, prec="w4a8")
    inp = generate(cfg, seed=14)
    for key in ("w1_bscale", "w2_bscale"):
        sc = torch.from_numpy(inp[key]).view(torch.float8_e4m3fn).to(torch.float32).numpy()
        assert np.isfinite(sc).all() and (6 * sc <= 448).all() and (sc >= 0).all()
    xs = inp["x_scale"]
    xq = torch.from_numpy(inp["x"]).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.abs(xq).max() <= 448 and xs.shape == (4, 2)


# ----------------------------------------------------------------------------- MXFP4 weights

def test_e8m0_is_a_power_of_two_with_bias_127():
    # OCP MX scale format: exponent only, bias 127, code 0xFF is NaN
    assert oracle.e8m0_value(127) == 1.0 and oracle.e8m0_value(128) == 2.0 and oracle.e8m0_value(126) == 0.5
    assert oracle.e8m0_value(0) == 2.0 ** -127 and oracle.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_value(255))


def test_mxfp4_values_in_the_required_scale_range_are_exact_in_fp8():
    # FlashInfer #6517 keeps MXFP4 scales within 2^-5..2^6 so that an FP8 decode neither saturates
    # nor flushes: there every exact MX value (the oracle's reading) is an e4m3 value
    for sc in range(122, 134):
        for c in range(16):
            v = oracle.e2m1_value(c) * oracle.e8m0_value(sc)
            assert oracle.e4m3_value(oracle.e4m3_encode(v)) == v
    assert oracle.e4m3_value(oracle.e4m3_encode(6 * 2.0 ** 7)) == 448.0  # one step above: saturates


def _mx_as_nvfp4(inp):
    """The same weights with each e8m0 block scale (one per 32 along K) written as the two equal
    e4m3 scales of its 16-wide halves: inside 2^-5..2^6 every e2m1 * scale product is an e4m3
    value, so the NVFP4 FP8 dequant reproduces the MX values exactly."""
    out = dict(inp)
    for key in ("w1_bscale", "w2_bscale"):
        v = np.ldexp(np.float32(1.0), inp[key].astype(np.int32) - 127).astype(np.float32)
        out[key] = torch.from_numpy(np.repeat(v, 2, axis=-1)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    out["cfg"] = dataclasses.replace(inp["cfg"], prec="w4a8")
    return out


def test_mxfp4_ffn_and_forward_equal_nvfp4_with_equal_block_scales():
    cfg = MoeConfig("t", T=6, H=256, I=256, E=3, k=2, prec="w4a8_mx", swiglu_clamp=10.0)
    inp = generate(cfg, seed=21)
    assert inp["w1_bscale"].shape == (3, 512, 8) and inp["w2_bscale"].shape == (3, 256, 8)
    rng = np.random.default_rng(5)  # scales varying block to block: a wrong block index changes values
    for key in ("w1_bscale", "w2_bscale"):
        inp[key] = rng.integers(122, 134, size=inp[key].shape).astype(np.uint8)
    nv = _mx_as_nvfp4(inp)
    tok = np.array([0, 1, 2, 3, 4, 5, 0, 3], np.int32)
    ex = np.array([0, 1, 2, 0, 1, 2, 2, 1], np.int32)
    assert np.array_equal(oracle.ffn_rows(inp, tok, ex), oracle.ffn_rows(nv, tok, ex))
    assert np.array_equal(oracle.moe_forward(inp), oracle.moe_forward(nv))


def test_mxfp4_ffn_equals_dense_computation_on_exact_weights():
    cfg = MoeConfig("t", T=5, H=256, I=256, E=2, k=2, prec="w4a8_mx", swiglu_clamp=10.0)
    inp = generate(cfg, seed=22)
    tok = np.array([0, 1, 2, 3, 4], np.int32)
    ex = np.array([0, 1, 1, 0, 1], np.int32)
    y = oracle.ffn_rows(inp, tok, ex)
    xq = torch.from_numpy(inp["x"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xd = xq * np.repeat(inp["x_scale"].astype(np.float64), 128, axis=1)

    def dense(packed, bscale, gscale):
        codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[0], -1)
        mag = E2M1_VALUES[codes & 7] * np.where(codes & 8, -1.0, 1.0)
        return mag * np.ldexp(1.0, np.repeat(bscale.astype(np.int64) - 127, 32, axis=1)) * np.float64(gscale)

    for i, (t, e) in enumerate(zip(tok, ex)):
        w1 = dense(inp["w1"][e], inp["w1_bscale"][e], inp["w1_gscale"][e])
        w2 = dense(inp["w2"][e], inp["w2_bscale"][e], inp["w2_gscale"][e])
        g = np.clip(xd[t] @ w1[: cfg.I].T, -10, 10)
        u = np.clip(xd[t] @ w1[cfg.I:].T, -10, 10)
        h = (g * scipy.special.expit(g) * u).astype(np.float32).reshape(-1, 128)
        s = (np.abs(h).max(axis=1) / np.float32(448)).astype(np.float32)
        s[s == 0] = 1
        hq = _torch_fp8_round((h / s[:, None]).astype(np.float32)) * s[:, None].astype(np.float64)
        np.testing.assert_allclose(y[i], hq.reshape(-1) @ w2.T, rtol=1e-9, atol=1e-12)


def _w4_dense(packed, bscale, gscale, mx):
    """one expert matrix, dequantised in numpy/torch: NVFP4 through torch's fp8 cast of the exact
    e2m1 * e4m3 product, MXFP4 exactly (e2m1 * 2^(e8m0 - 127)); times the global scale"""
    if not mx:
        return _dequant_nvfp4(packed, bscale, gscale)
    codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(packed.shape[0], -1)
    mag = E2M1_VALUES[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    return mag * np.ldexp(1.0, np.repeat(bscale.astype(np.int64) - 127, 32, axis=1)) * np.float64(gscale)


def _w4a8_forward_dense(inp, swap01=False):
    """The W4A8 forward token by token: scipy softmax over the logits, the k largest (stable
    argsort), renormalised over them, dropped slots skipped; each expert as dense numpy matrices
    (W1 rows de-interleaved), h re-quantised per 128 with torch's fp8 cast.  swap01 pairs the
    weights of slots 0 and 1 the wrong way round (to show the comparison would see it)."""
    cfg = inp["cfg"]
    mx = cfg.prec == "w4a8_mx"
    xq = torch.from_numpy(inp["x"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    xd = xq * np.repeat(inp["x_scale"].astype(np.float64), 128, axis=1)
    w1 = [deinterleave_rows(_w4_dense(inp["w1"][e], inp["w1_bscale"][e], inp["w1_gscale"][e], mx), cfg.I,
                            cfg.glu_interleave) for e in range(cfg.E)]
    w2 = [_w4_dense(inp["w2"][e], inp["w2_bscale"][e], inp["w2_gscale"][e], mx) for e in range(cfg.E)]
    out = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        p = scipy.special.softmax(inp["logits"][t].astype(np.float64))
        sel = np.argsort(-p, kind="stable")[: cfg.k]
        w = p[sel] / p[sel].sum()
        if swap01:
            w[[0, 1]] = w[[1, 0]]
        for j, e in enumerate(sel):
            if inp["slot_drop"] is not None and inp["slot_drop"][t, j]:
                continue
            c = cfg.swiglu_clamp
            g, u = xd[t] @ w1[e][: cfg.I].T, xd[t] @ w1[e][cfg.I:].T
            if c:
                g, u = np.clip(g, -c, c), np.clip(u, -c, c)
            h = (g * scipy.special.expit(g) * u).astype(np.float32).reshape(-1, 128)
            s = (np.abs(h).max(axis=1) / np.float32(448)).astype(np.float32)
            s[s == 0] = 1
            hq = _torch_fp8_round((h / s[:, None]).astype(np.float32)) * s[:, None].astype(np.float64)
            out[t] += w[j] * (hq.reshape(-1) @ w2[e].T)
    return out


@pytest.mark.parametrize("prec", ["w4a8", "w4a8_mx"])
def test_w4a8_forward_equals_routed_weighted_dense_computation(prec):
    """the W4A8 / MXFP4 branch of the oracle's forward (routing, expert choice, weights, dropped
    slots, interleaved W1, clamp, h re-quantisation, combine) against the dense numpy computation"""
    cfg = MoeConfig("t", T=12, H=256, I=256, E=5, k=3, prec=prec, glu_interleave=32, swiglu_clamp=10.0,
                    drop_p=0.25)
    inp = generate(cfg, seed=41)
    assert inp["slot_drop"].any() and not inp["slot_drop"].all()
    got = oracle.moe_forward(inp)
    want = _w4a8_forward_dense(inp)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)
    # a mispaired combine (weights of slots 0 and 1 exchanged) is far outside that tolerance
    assert np.abs(_w4a8_forward_dense(inp, swap01=True) - got).max() > 1e-3 * np.abs(got).max()


def test_mxfp4_generator_keeps_scales_in_the_required_range():
    # FlashInfer #6517: MXFP4 block scales within 2^-5..2^6; the rest in a power-of-two global scale
    cfg = MoeConfig("t", T=4, H=512, I=256, E=2, k=1, prec="w4a8_mx")
    inp = generate(cfg, seed=23)
    for key in ("w1_bscale", "w2_bscale"):
        assert (inp[key] >= 122).all() and (inp[key] <= 133).all() and (inp[key] == 133).any()
    for key in ("w1_gscale", "w2_gscale"):
        m, _ = np.frexp(inp[key])
        assert (m == 0.5).all()  # powers of two


# ----------------------------------------------------------------------------- generator

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3e38, -0.0], np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bf16_bits_from_f32(v) == want).all()


def test_interleave_layout_definition():
    perm = _interleave_perm(128, 32)
    assert list(perm[:4]) == [0, 1, 2, 3] and perm[32] == 128 and perm[63] == 159 and perm[64] == 32
    assert sorted(perm) == list(range(256))


def test_generator_is_prefix_stable_in_T():
    a = generate(CONFIGS["ep_share"], seed=3, T=64, weights=False)
    b = generate(CONFIGS["ep_share"], seed=3, T=128, weights=False)
    assert (a["x"] == b["x"][:64]).all() and (a["logits"] == b["logits"][:64]).all()
    assert (a["slot_drop"] == b["slot_drop"][:64]).all()
