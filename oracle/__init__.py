"""CPU oracle for the MoE FFN forward -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under test never does, and
this package imports nothing from it.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64, one token at a time);
this module builds it with gcc and wraps it for numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile moe_oracle.c -> liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = f64
    lib.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1_value.restype = f64
    lib.orc_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.orc_e8m0_value.restype = f64
    lib.orc_e4m3_encode.argtypes = [f64]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_fp4_to_fp8.argtypes = [ctypes.c_uint8, ctypes.c_uint8]
    lib.orc_fp4_to_fp8.restype = ctypes.c_uint8
    lib.orc_route.argtypes = [i32, i32, i32, P, P, P, P]
    lib.orc_tables.argtypes = [i32, i32, i32, P, P, P, P, P]
    lib.orc_permute_rows.argtypes = [i64, i32, i32, P, P, P]
    lib.orc_combine_bf16.argtypes = [i32, i32, i32, P, P, P, P]
    lib.orc_ffn_rows_bf16.argtypes = [i64, P, P, i32, i32, i32, f64, P, P, P, P]
    lib.orc_ffn_rows_w4a8.argtypes = [i64, P, P, i32, i32, i32, f64, P, P, P, P, P, P, P, P, i32, P]
    lib.orc_moe_forward.argtypes = [i32, P, i32, i32, i32, i32, i32, i32, i32, f64,
                                    P, P, P, P, P, P, P, P, P, P, P]
    lib.orc_max_threads.restype = i32
    lib.orc_set_threads.argtypes = [i32]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats

def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e8m0_value(code: int) -> float:
    return _load().orc_e8m0_value(int(code))


def e4m3_encode(v: float) -> int:
    return int(_load().orc_e4m3_encode(float(v)))


def fp4_to_fp8(code4: int, scale8: int) -> int:
    return int(_load().orc_fp4_to_fp8(int(code4), int(scale8)))


def fp4_to_fp8_table() -> np.ndarray:
    """uint8 [16][256]: the fp8 code of every (e2m1 code, e4m3 block scale) pair."""
    lib = _load()
    return np.array([[lib.orc_fp4_to_fp8(c, s) for s in range(256)] for c in range(16)], dtype=np.uint8)


# ---------------------------------------------------------------- steps

def route(logits, k, slot_drop=None):
    """-> (topk_idx int32 [T][k], topk_w float64 [T][k])"""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    dr = _c(slot_drop, np.uint8)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _load().orc_route(T, E, k, _p(lg), _p(dr), _p(idx), _p(w))
    return idx, w


def tables(topk_idx, E):
    """-> (counts [E], offsets [E+1], row_src [T*k], slot_row [T*k]) int32"""
    idx = _c(topk_idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_src = np.empty(T * k, np.int32)
    slot_row = np.empty(T * k, np.int32)
    _load().orc_tables(T, k, E, _p(idx), _p(counts), _p(offsets), _p(row_src), _p(slot_row))
    return counts, offsets, row_src, slot_row


def permute_rows(x, row_src, R, k):
    x = _c(x, np.uint16)
    rs = _c(row_src, np.int32)
    H = x.shape[1]
    out = np.empty((R, H), np.uint16)
    _load().orc_permute_rows(R, k, H, _p(rs), _p(x), _p(out))
    return out


def combine_bf16(y_perm, slot_row, topk_w, T, k):
    y = _c(y_perm, np.uint16)
    sr = _c(slot_row, np.int32)
    w = _c(topk_w, np.float32)
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    _load().orc_combine_bf16(T, k, H, _p(y), _p(sr), _p(w), _p(out))
    return out


class _Keep:
    """Holds the contiguous copies handed to C until the call returns."""

    def __init__(self):
        self.refs = []

    def __call__(self, a, dtype):
        a = _c(a, dtype)
        self.refs.append(a)
        return _p(a)


def ffn_rows(inp: dict, tokens, experts):
    """y[i] = FFN_{experts[i]}(x[tokens[i]]) in fp64, for either precision."""
    cfg = inp["cfg"]
    keep = _Keep()
    tok = _c(tokens, np.int32)
    ex = _c(experts, np.int32)
    n = tok.size
    y = np.empty((n, cfg.H), np.float64)
    lib = _load()
    if cfg.prec == "bf16":
        lib.orc_ffn_rows_bf16(n, _p(tok), _p(ex), cfg.H, cfg.I, cfg.glu_interleave, cfg.swiglu_clamp,
                              keep(inp["x"], np.uint16), keep(inp["w1"], np.uint16),
                              keep(inp["w2"], np.uint16), _p(y))
    else:
        lib.orc_ffn_rows_w4a8(n, _p(tok), _p(ex), cfg.H, cfg.I, cfg.glu_interleave, cfg.swiglu_clamp,
                              keep(inp["x"], np.uint8), keep(inp["x_scale"], np.float32),
                              keep(inp["w1"], np.uint8), keep(inp["w1_bscale"], np.uint8),
                              keep(inp["w1_gscale"], np.float32), keep(inp["w2"], np.uint8),
                              keep(inp["w2_bscale"], np.uint8), keep(inp["w2_gscale"], np.float32),
                              1 if cfg.prec == "w4a8_mx" else 0, _p(y))
    return y


def moe_forward(inp: dict, tokens=None):
    """out[i] = sum_j w_j FFN_{e_j}(x[t_i]) in fp64 for the listed tokens (all if None)."""
    cfg = inp["cfg"]
    if tokens is None:
        tokens = np.arange(cfg.T, dtype=np.int32)
    keep = _Keep()
    tok = _c(tokens, np.int32)
    out = np.empty((tok.size, cfg.H), np.float64)
    w4 = cfg.prec != "bf16"
    xdt = np.uint8 if w4 else np.uint16
    prec = {"bf16": 0, "w4a8": 1, "w4a8_mx": 2}[cfg.prec]
    _load().orc_moe_forward(
        tok.size, _p(tok), cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, prec, cfg.glu_interleave,
        cfg.swiglu_clamp, keep(inp["logits"], np.float32), keep(inp.get("slot_drop"), np.uint8),
        keep(inp["x"], xdt), keep(inp.get("x_scale"), np.float32),
        keep(inp["w1"], xdt), keep(inp.get("w1_bscale"), np.uint8),
        keep(inp.get("w1_gscale"), np.float32), keep(inp["w2"], xdt),
        keep(inp.get("w2_bscale"), np.uint8), keep(inp.get("w2_gscale"), np.float32), _p(out))
    return out


def max_threads() -> int:
    return _load().orc_max_threads()


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))
