"""MI355X-native Mixture-of-Experts FFN forward: Python binding of libtpg_moe.so.

The functions here carry the C ABI's names (include/moe.h) and do argument
marshalling only: tensors become device pointers, the stream defaults to torch's
current stream, and a non-zero status raises MoeError.  Every step of the forward
runs in the library's HIP kernels; there is no fallback.  If the library has not
been built, importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpg_moe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_SCRATCH = range(7)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_PREC_BF16, MOE_PREC_W4A8, MOE_PREC_W4A8_MX = 0, 1, 2
# precision of a synthetic workload's `prec` name
PRECISIONS = {"bf16": MOE_PREC_BF16, "w4a8": MOE_PREC_W4A8, "w4a8_mx": MOE_PREC_W4A8_MX}
MOE_W4_LAYOUT_ROWS, MOE_W4_LAYOUT_TILED = 0, 1
MOE_WS_PERMUTE, MOE_WS_GROUPED_FFN, MOE_WS_FORWARD = 0, 1, 2

# every symbol include/moe.h declares
EXPORTS = (
    "moe_workspace_bytes", "moe_call_workspace_bytes", "moe_status_str", "moe_last_hip_error", "moe_route_topk", "moe_permute",
    "moe_permute_timed", "moe_grouped_ffn", "moe_unpermute_combine", "moe_forward", "moe_forward_timed", "moe_forward_noalloc", "moe_w4a8_dequant_table",
    "moe_w4a8_tile_weights",
)
MOE_N_STAGE_EVENTS = 8
MOE_N_PERMUTE_EVENTS = 3
STAGES = ("route", "tables", "gather", "tile_list", "gemm1_swiglu", "gemm2", "combine")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str, hip: int = 0):
        super().__init__(f"{fn}: {text} (status {status}{', hipError ' + str(hip) if hip else ''})")
        self.status = status
        self.hip_error = hip


MOE_FLAG_SINGLE_LAUNCH = 1
MOE_FLAG_SCATTER_Y = 2


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("prec", ctypes.c_int32), ("glu_interleave", ctypes.c_int32),
                ("swiglu_clamp", ctypes.c_float), ("flags", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("w1_bscale", ctypes.c_void_p), ("w1_gscale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_bscale", ctypes.c_void_p), ("w2_gscale", ctypes.c_void_p),
                ("w4_layout", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libtpg_moe.so (built in-tree by token_permute_grouped_amd._build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m token_permute_grouped_amd._build` "
                          "(or __graft_entry__.build()); there is no fallback path")
    # torch first: it carries the process's HIP runtime (same SONAME as the one this library links), so
    # torch's streams and allocations and this library's launches share one runtime instance
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    PP = ctypes.POINTER(Problem)
    PW = ctypes.POINTER(Weights)
    lib.moe_workspace_bytes.argtypes = [PP]
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_call_workspace_bytes.argtypes = [PP, I32]
    lib.moe_call_workspace_bytes.restype = SZ
    lib.moe_status_str.argtypes = [I32]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_last_hip_error.restype = I32
    lib.moe_route_topk.argtypes = [P, P, PP, P, P, P]
    lib.moe_permute.argtypes = [P, P, P, PP, P, P, P, P, P, P, SZ, P]
    lib.moe_permute_timed.argtypes = [P, P, P, PP, P, P, P, P, P, P, SZ, P, ctypes.POINTER(ctypes.c_void_p)]
    lib.moe_grouped_ffn.argtypes = [P, P, P, PW, PP, P, P, SZ, P]
    lib.moe_unpermute_combine.argtypes = [P, P, P, PP, P, P]
    lib.moe_forward.argtypes = [P, P, P, P, PW, PP, P, P, SZ, P]
    lib.moe_forward_timed.argtypes = [P, P, P, P, PW, PP, P, P, SZ, P, ctypes.POINTER(ctypes.c_void_p)]
    lib.moe_forward_noalloc.argtypes = [P, P, P, P, PW, PP, P, P]
    lib.moe_w4a8_dequant_table.argtypes = [P, P]
    lib.moe_w4a8_tile_weights.argtypes = [P, P, P, P, I32, I32, I32, I32, P]
    for name in ("moe_route_topk", "moe_permute", "moe_permute_timed", "moe_grouped_ffn", "moe_unpermute_combine", "moe_forward",
                 "moe_forward_timed", "moe_forward_noalloc", "moe_w4a8_dequant_table", "moe_w4a8_tile_weights"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib


def _ptr(t):
    """None -> NULL, int -> itself, tensor -> its device address."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    if t is None:
        return 0
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int):
    if st != MOE_OK:
        lib = load()
        raise MoeError(fn, st, lib.moe_status_str(st).decode(), lib.moe_last_hip_error() if st == MOE_ERR_HIP else 0)


def make_problem(T, H, I, E, k, prec=MOE_PREC_BF16, glu_interleave=0, swiglu_clamp=0.0, flags=0) -> Problem:
    return Problem(T, H, I, E, k, prec, glu_interleave, swiglu_clamp, flags)


def make_weights(w1, w2, w1_bscale=None, w1_gscale=None, w2_bscale=None, w2_gscale=None,
                 w4_layout=MOE_W4_LAYOUT_ROWS) -> Weights:
    return Weights(_ptr(w1), _ptr(w1_bscale), _ptr(w1_gscale), _ptr(w2), _ptr(w2_bscale), _ptr(w2_gscale),
                   w4_layout)


def moe_workspace_bytes(problem: Problem) -> int:
    """bytes of workspace that serve every entry point (moe_forward's plan)"""
    return int(load().moe_workspace_bytes(ctypes.byref(problem)))


def moe_call_workspace_bytes(problem: Problem, which: int) -> int:
    """the smaller workspace of one step entry point (MOE_WS_PERMUTE / MOE_WS_GROUPED_FFN)"""
    return int(load().moe_call_workspace_bytes(ctypes.byref(problem), which))


def moe_route_topk(logits, slot_drop, problem: Problem, topk_idx, topk_w, stream=None):
    _check("moe_route_topk", load().moe_route_topk(_ptr(logits), _ptr(slot_drop), ctypes.byref(problem),
                                                   _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def moe_permute(x, x_scale, topk_idx, problem: Problem, offsets, row_src, slot_row, x_perm, x_perm_scale, ws,
                ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    _check("moe_permute", load().moe_permute(_ptr(x), _ptr(x_scale), _ptr(topk_idx), ctypes.byref(problem),
                                             _ptr(offsets), _ptr(row_src), _ptr(slot_row), _ptr(x_perm),
                                             _ptr(x_perm_scale), _ptr(ws), ws_bytes, _stream(stream)))


def moe_permute_timed(x, x_scale, topk_idx, problem: Problem, offsets, row_src, slot_row, x_perm, x_perm_scale, ws,
                      stage_events, ws_bytes=None, stream=None):
    """stage_events: MOE_N_PERMUTE_EVENTS raw hipEvent_t handles (ints)"""
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    ev = (ctypes.c_void_p * MOE_N_PERMUTE_EVENTS)(*stage_events)
    _check("moe_permute_timed", load().moe_permute_timed(_ptr(x), _ptr(x_scale), _ptr(topk_idx),
                                                         ctypes.byref(problem), _ptr(offsets), _ptr(row_src),
                                                         _ptr(slot_row), _ptr(x_perm), _ptr(x_perm_scale), _ptr(ws),
                                                         ws_bytes, _stream(stream), ev))


def moe_grouped_ffn(x_perm, x_perm_scale, offsets, weights: Weights, problem: Problem, y_perm, ws, ws_bytes=None,
                    stream=None):
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    _check("moe_grouped_ffn", load().moe_grouped_ffn(_ptr(x_perm), _ptr(x_perm_scale), _ptr(offsets),
                                                     ctypes.byref(weights), ctypes.byref(problem), _ptr(y_perm),
                                                     _ptr(ws), ws_bytes, _stream(stream)))


def moe_unpermute_combine(y_perm, slot_row, topk_w, problem: Problem, out, stream=None):
    _check("moe_unpermute_combine", load().moe_unpermute_combine(_ptr(y_perm), _ptr(slot_row), _ptr(topk_w),
                                                                 ctypes.byref(problem), _ptr(out), _stream(stream)))


def moe_forward(logits, slot_drop, x, x_scale, weights: Weights, problem: Problem, out, ws, ws_bytes=None,
                stream=None):
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    _check("moe_forward", load().moe_forward(_ptr(logits), _ptr(slot_drop), _ptr(x), _ptr(x_scale),
                                             ctypes.byref(weights), ctypes.byref(problem), _ptr(out), _ptr(ws),
                                             ws_bytes, _stream(stream)))


def moe_forward_timed(logits, slot_drop, x, x_scale, weights: Weights, problem: Problem, out, ws, stage_events,
                      ws_bytes=None, stream=None):
    """stage_events: MOE_N_STAGE_EVENTS raw hipEvent_t handles (ints)"""
    if ws_bytes is None:
        ws_bytes = _nbytes(ws)
    ev = (ctypes.c_void_p * MOE_N_STAGE_EVENTS)(*stage_events)
    _check("moe_forward_timed", load().moe_forward_timed(_ptr(logits), _ptr(slot_drop), _ptr(x), _ptr(x_scale),
                                                         ctypes.byref(weights), ctypes.byref(problem), _ptr(out),
                                                         _ptr(ws), ws_bytes, _stream(stream), ev))


def moe_forward_noalloc(logits, slot_drop, x, x_scale, weights: Weights, problem: Problem, out, stream=None):
    """moe_forward on the library's own device scratch (no workspace argument, nothing allocated)"""
    _check("moe_forward_noalloc", load().moe_forward_noalloc(_ptr(logits), _ptr(slot_drop), _ptr(x), _ptr(x_scale),
                                                             ctypes.byref(weights), ctypes.byref(problem), _ptr(out),
                                                             _stream(stream)))


def moe_w4a8_tile_weights(codes, bscale, codes_tiled, bscale_tiled, E, N, K, prec, stream=None):
    """row-major W4A8 codes [E][N][K/2] and block scales -> MOE_W4_LAYOUT_TILED (see include/moe.h)"""
    _check("moe_w4a8_tile_weights", load().moe_w4a8_tile_weights(_ptr(codes), _ptr(bscale), _ptr(codes_tiled),
                                                                 _ptr(bscale_tiled), E, N, K, prec, _stream(stream)))


def moe_w4a8_dequant_table(out8, stream=None):
    """out8: device uint8 [8][16][256] (see include/moe.h)."""
    if _nbytes(out8) < 8 * 16 * 256:
        raise ValueError("moe_w4a8_dequant_table needs an 8*16*256-byte output")
    _check("moe_w4a8_dequant_table", load().moe_w4a8_dequant_table(_ptr(out8), _stream(stream)))
