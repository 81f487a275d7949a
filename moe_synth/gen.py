"""Seeded generator for the MoE FFN forward workloads.

Workloads (sizes and value distributions as the task's configurations give them):

* ``tiny``      T=64,    H=128,  I=256,  E=8,   top-2, bf16.
* ``mid``       T=4096,  H=2048, I=1408, E=64,  top-6, bf16.
* ``skewed``    T=16384, H=4096, I=2048, E=128, top-8, bf16; router logits carry a
                per-expert bias so that expert popularity follows Zipf s=1.2.
* ``w4a8``      T in {1..256}, H=7168, I=2048, E=32, top-8; fp8 e4m3 activations
                with one fp32 scale per 128 columns, NVFP4 weights (e2m1 codes,
                one e4m3 scale per 16 elements along K, one fp32 global scale per
                expert and matrix); SwiGLU input clamped to +-10.
* ``w4a8_mx``   as ``w4a8`` with MXFP4 weights: e2m1 codes, one e8m0 (power-of-two)
                scale per 32 elements along K, one fp32 global scale per expert
                and matrix.
* ``ep_share``  T=32768, H=7168, I=2048, E=32, top-8, bf16; W1 gate/up rows
                interleaved in blocks of 32; 10% of (token, slot) pairs dropped.

Distributions: x ~ N(0,1); W1 ~ N(0, H^-1/2) and W2 ~ N(0, I^-1/2) (standard
deviation fan_in^-1/2); router logits ~ N(0,1) fp32.

Random streams: ``SeedSequence(seed).spawn`` gives one independent child per
tensor, and per-expert grandchildren for the weights, so values do not depend on
generation order, on threading, or (for x, logits and the drop mask) on T beyond
the rows drawn: the first T' rows of a T-row draw equal a T'-row draw.

Layouts (all row-major, K contiguous):
  x         bf16 bits uint16 [T][H]            | w4a8: e4m3 codes uint8 [T][H] + f32 [T][H/128]
  logits    float32 [T][E]
  slot_drop uint8 [T][k] (1 = slot routed to no local expert) or None
  w1        bf16 bits uint16 [E][2I][H]        | w4a8: uint8 [E][2I][H/2] (low nibble = even k)
                                                   + e4m3 uint8 [E][2I][H/16] + f32 [E]
  w2        bf16 bits uint16 [E][H][I]         | w4a8: uint8 [E][H][I/2] + uint8 [E][H][I/16] + f32 [E]
                                               | w4a8_mx: block scales e8m0 uint8 [E][2I][H/32], [E][H][I/32]
W1 rows are [gate | up] (gate rows 0..I-1), or, with an interleave of 32, stored
row 64q+r holds gate row 32q+r for r<32 and up row 32q+r-32 for r>=32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

try:  # torch is used only for its fp8 e4m3fn cast when encoding w4a8 inputs
    import torch
except Exception:  # pragma: no cover - torch is present in every supported image
    torch = None


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    prec: str = "bf16"          # "bf16", "w4a8" (NVFP4 weights) or "w4a8_mx" (MXFP4 weights)
    glu_interleave: int = 0     # 0 = [gate|up]; 32 = 32-row blocks gate,up,gate,up,...
    swiglu_clamp: float = 0.0   # 0 = none; c>0 clamps gate and up to [-c, c]
    zipf_s: float = 0.0         # >0: per-expert logit bias ln(rank^-s)
    drop_p: float = 0.0         # probability that a (token, slot) pair is dropped

    def with_tokens(self, T: int) -> "MoeConfig":
        return replace(self, T=T)

    @property
    def flops(self) -> int:
        """Dense-equivalent flops of the two grouped GEMMs for all T*k slots."""
        return 6 * self.T * self.k * self.H * self.I


CONFIGS = {
    "tiny": MoeConfig("tiny", T=64, H=128, I=256, E=8, k=2),
    "mid": MoeConfig("mid", T=4096, H=2048, I=1408, E=64, k=6),
    "skewed": MoeConfig("skewed", T=16384, H=4096, I=2048, E=128, k=8, zipf_s=1.2),
    "w4a8": MoeConfig("w4a8", T=256, H=7168, I=2048, E=32, k=8, prec="w4a8",
                      swiglu_clamp=10.0),
    "w4a8_mx": MoeConfig("w4a8_mx", T=256, H=7168, I=2048, E=32, k=8, prec="w4a8_mx",
                         swiglu_clamp=10.0),
    "ep_share": MoeConfig("ep_share", T=32768, H=7168, I=2048, E=32, k=8,
                          glu_interleave=32, drop_p=0.1),
}


def w4a8_sweep_tokens():
    return [1, 2, 4, 8, 16, 32, 64, 128, 256]


# ----------------------------------------------------------------------------
# bf16 bit encoding (input preparation)
# ----------------------------------------------------------------------------

def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# gate/up row layout
# ----------------------------------------------------------------------------

def _interleave_perm(I: int, il: int) -> np.ndarray:
    """perm[p] = logical [gate|up] row stored at physical row p."""
    p = np.arange(2 * I)
    q, r = p // (2 * il), p % (2 * il)
    return np.where(r < il, q * il + r, I + q * il + (r - il))


def interleave_rows(w1_logical: np.ndarray, I: int, il: int) -> np.ndarray:
    """[.., 2I, K] in [gate|up] order -> stored order for interleave ``il`` (0 = unchanged)."""
    if il == 0:
        return w1_logical
    return np.ascontiguousarray(w1_logical[..., _interleave_perm(I, il), :])


def deinterleave_rows(w1_stored: np.ndarray, I: int, il: int) -> np.ndarray:
    if il == 0:
        return w1_stored
    inv = np.empty(2 * I, dtype=np.int64)
    inv[_interleave_perm(I, il)] = np.arange(2 * I)
    return np.ascontiguousarray(w1_stored[..., inv, :])


# ----------------------------------------------------------------------------
# fp8 / fp4 input encoders (input preparation for the w4a8 workload)
# ----------------------------------------------------------------------------

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _e4m3_codes(v: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn codes, round to nearest even, saturating at +-448."""
    t = torch.from_numpy(np.clip(np.ascontiguousarray(v, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_decode(c: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(c, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def _e2m1_codes(v: np.ndarray) -> np.ndarray:
    """float32 -> e2m1 codes (sign bit 3), round to nearest even, saturating at +-6.

    The magnitude code is the number of midpoints between neighbouring e2m1 values
    that lie strictly below |v|; a value exactly on a midpoint goes to the even code.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v)
    idx = np.zeros(v.shape, dtype=np.uint8)
    for j, m in enumerate(_E2M1_MIDS):
        idx += a > m
        if j % 2 == 1:          # a tie at an odd midpoint rounds up to the even code j + 1
            idx += a == m
    sign = (np.signbit(v) & (idx > 0)).astype(np.uint8)
    return idx | (sign << np.uint8(3))


def _quantise_act_rows(xf: np.ndarray):
    """x fp32 [T][H] -> (e4m3 codes [T][H], fp32 scales [T][H/128]); s = amax/448 per 128."""
    T, H = xf.shape
    blk = xf.reshape(T, H // 128, 128)
    amax = np.abs(blk).max(axis=2).astype(np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    q = _e4m3_codes((blk / s[:, :, None]).astype(np.float32)).reshape(T, H)
    return q, s


def _quantise_nvfp4(w: np.ndarray):
    """One expert's matrix fp32 [N][K] -> (packed e2m1 [N][K/2], e4m3 scales [N][K/16], fp32 global).

    gs = amax/448; block scale = e4m3(amax_16 / (6 gs)); code = e2m1(w / (scale gs)).
    """
    N, K = w.shape
    # block scales stay inside the fp8 decoder range (6 * scale <= 448): the largest block
    # scale is amax/(6 gs) = 448/6, which rounds to 72 in e4m3; the rest goes into gs.
    gs = np.float32(np.abs(w).max() / 448.0)
    if gs == 0:
        gs = np.float32(1.0)
    packed = np.empty((N, K // 2), dtype=np.uint8)
    bs_code = np.empty((N, K // 16), dtype=np.uint8)
    for r0 in range(0, N, 256):  # row blocks keep the temporaries small
        blk = w[r0:r0 + 256].reshape(-1, K // 16, 16)
        amax16 = np.abs(blk).max(axis=2).astype(np.float32)
        bc = _e4m3_codes((amax16 / (np.float32(6.0) * gs)).astype(np.float32))
        denom = (_e4m3_decode(bc).astype(np.float32) * gs)[:, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(denom > 0, blk / np.where(denom > 0, denom, 1), 0).astype(np.float32)
        codes = _e2m1_codes(ratio).reshape(-1, K)
        packed[r0:r0 + 256] = codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))
        bs_code[r0:r0 + 256] = bc
    return packed, bs_code, gs


def _quantise_mxfp4(w: np.ndarray):
    """One expert's matrix fp32 [N][K] -> (packed e2m1 [N][K/2], e8m0 scales [N][K/32], fp32 global).

    The global scale is a power of two, gs = 2^(floor(log2 amax) - 8), so that a block holding the
    matrix's largest value gets block exponent 6.  Block exponent (OCP MX: floor(log2) of the
    block's amax minus e2m1's largest exponent, 2) eb = floor(log2(amax_32 / gs)) - 2, kept within
    -5..6 (the scale range the FlashInfer follow-up #6517 asks for); scale code eb + 127; code =
    e2m1(w / (2^eb gs)), round to nearest even, saturating at +-6.
    """
    N, K = w.shape
    amax = float(np.abs(w).max())
    gs = np.float32(2.0 ** (np.floor(np.log2(amax)) - 8)) if amax > 0 else np.float32(1.0)
    packed = np.empty((N, K // 2), dtype=np.uint8)
    bs_code = np.empty((N, K // 32), dtype=np.uint8)
    for r0 in range(0, N, 256):  # row blocks keep the temporaries small
        blk = w[r0:r0 + 256].reshape(-1, K // 32, 32)
        amax32 = np.abs(blk).max(axis=2).astype(np.float64)
        with np.errstate(divide="ignore"):
            eb = np.floor(np.log2(amax32 / float(gs))) - 2
        eb = np.clip(np.where(amax32 > 0, eb, -5), -5, 6).astype(np.int32)
        scale = (np.ldexp(np.float32(1.0), eb) * gs).astype(np.float32)
        codes = _e2m1_codes((blk / scale[:, :, None]).astype(np.float32)).reshape(-1, K)
        packed[r0:r0 + 256] = codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))
        bs_code[r0:r0 + 256] = (eb + 127).astype(np.uint8)
    return packed, bs_code, gs


# ----------------------------------------------------------------------------
# the generator
# ----------------------------------------------------------------------------

def _normal(seed_seq, n, dtype=np.float32):
    return np.random.Generator(np.random.PCG64(seed_seq)).standard_normal(n, dtype=dtype)


def _threads(threads):
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def generate(cfg: MoeConfig, seed: int = 0, T: int | None = None, threads: int | None = None,
             weights: bool = True) -> dict:
    """Draw every input of one workload. Returns a dict of numpy arrays (see module doc)."""
    if T is not None:
        cfg = cfg.with_tokens(T)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    ss = np.random.SeedSequence(seed)
    c_x, c_logit, c_bias, c_w1, c_w2, c_drop = ss.spawn(6)
    out: dict = {"cfg": cfg, "seed": seed}

    # router logits: N(0,1) (+ Zipf bias), fp32
    lg = np.random.Generator(np.random.PCG64(c_logit)).standard_normal((T, E), dtype=np.float64)
    if cfg.zipf_s > 0:
        ranks = np.random.Generator(np.random.PCG64(c_bias)).permutation(E) + 1
        lg = lg + (-cfg.zipf_s * np.log(ranks.astype(np.float64)))[None, :]
        out["expert_rank"] = ranks.astype(np.int32)
    out["logits"] = np.ascontiguousarray(lg.astype(np.float32))

    out["slot_drop"] = None
    if cfg.drop_p > 0:
        u = np.random.Generator(np.random.PCG64(c_drop)).random((T, k))
        out["slot_drop"] = np.ascontiguousarray((u < cfg.drop_p).astype(np.uint8))

    xf = np.random.Generator(np.random.PCG64(c_x)).standard_normal((T, H), dtype=np.float32)
    if cfg.prec == "bf16":
        out["x"] = bf16_bits_from_f32(xf).reshape(T, H)
    else:
        out["x"], out["x_scale"] = _quantise_act_rows(xf)

    if not weights:
        return out

    ch1 = c_w1.spawn(E)
    ch2 = c_w2.spawn(E)
    sd1 = np.float32(1.0 / np.sqrt(H))
    sd2 = np.float32(1.0 / np.sqrt(I))
    perm = _interleave_perm(I, cfg.glu_interleave) if cfg.glu_interleave else None

    if cfg.prec == "bf16":
        w1 = np.empty((E, 2 * I, H), dtype=np.uint16)
        w2 = np.empty((E, H, I), dtype=np.uint16)

        def job(e):
            a = (_normal(ch1[e], 2 * I * H) * sd1).reshape(2 * I, H)
            if perm is not None:
                a = a[perm]
            w1[e] = bf16_bits_from_f32(a).reshape(2 * I, H)
            b = (_normal(ch2[e], H * I) * sd2).reshape(H, I)
            w2[e] = bf16_bits_from_f32(b).reshape(H, I)

        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(job, range(E)))
        out["w1"], out["w2"] = w1, w2
    else:
        mx = cfg.prec == "w4a8_mx"
        bk = 32 if mx else 16  # K values per block scale
        quant = _quantise_mxfp4 if mx else _quantise_nvfp4
        w1 = np.empty((E, 2 * I, H // 2), dtype=np.uint8)
        w1b = np.empty((E, 2 * I, H // bk), dtype=np.uint8)
        w1g = np.empty(E, dtype=np.float32)
        w2 = np.empty((E, H, I // 2), dtype=np.uint8)
        w2b = np.empty((E, H, I // bk), dtype=np.uint8)
        w2g = np.empty(E, dtype=np.float32)

        def job(e):
            a = (_normal(ch1[e], 2 * I * H) * sd1).reshape(2 * I, H)
            if perm is not None:
                a = a[perm]
            w1[e], w1b[e], w1g[e] = quant(a)
            b = (_normal(ch2[e], H * I) * sd2).reshape(H, I)
            w2[e], w2b[e], w2g[e] = quant(b)

        with ThreadPoolExecutor(_threads(threads)) as ex:
            list(ex.map(job, range(E)))
        out.update(w1=w1, w1_bscale=w1b, w1_gscale=w1g, w2=w2, w2_bscale=w2b, w2_gscale=w2g)
    return out
