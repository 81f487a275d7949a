"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/moe.h declares, and reject
bad arguments on the host -- before anything is enqueued -- with the documented
status codes.  No test here launches a kernel: each call below fails a host check
(or has T == 0) and returns before any HIP call.
"""
import ctypes
import os
import re

import pytest

import token_permute_grouped_amd as tpg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call below returns on a host check first


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(moe_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    lib = tpg.load()
    declared = _declared_functions()
    assert declared == set(tpg.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def _p(**kw):
    base = dict(T=64, H=128, I=256, E=8, k=2, prec=0, glu_interleave=0, swiglu_clamp=0.0)
    base.update(kw)
    return tpg.Problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), tpg.MOE_ERR_SHAPE), (dict(H=100), tpg.MOE_ERR_SHAPE), (dict(H=0), tpg.MOE_ERR_SHAPE),
    (dict(I=64), tpg.MOE_ERR_SHAPE), (dict(E=0), tpg.MOE_ERR_SHAPE), (dict(E=257, k=2), tpg.MOE_ERR_SHAPE),
    (dict(k=0), tpg.MOE_ERR_SHAPE), (dict(k=9, E=8), tpg.MOE_ERR_SHAPE), (dict(k=65, E=64), tpg.MOE_ERR_SHAPE),
    (dict(k=257, E=256), tpg.MOE_ERR_SHAPE),
    (dict(T=2 ** 28, k=8), tpg.MOE_ERR_SHAPE), (dict(prec=7), tpg.MOE_ERR_UNSUPPORTED),
    (dict(glu_interleave=16), tpg.MOE_ERR_UNSUPPORTED), (dict(swiglu_clamp=-1.0), tpg.MOE_ERR_UNSUPPORTED),
    (dict(swiglu_clamp=float("nan")), tpg.MOE_ERR_UNSUPPORTED),
    (dict(prec=1, H=384), tpg.MOE_ERR_SHAPE), (dict(prec=1, I=384), tpg.MOE_ERR_SHAPE),
    (dict(prec=2, H=384), tpg.MOE_ERR_SHAPE), (dict(prec=2, I=384), tpg.MOE_ERR_SHAPE), (dict(prec=3), tpg.MOE_ERR_UNSUPPORTED),
    (dict(H=65536, I=8192), tpg.MOE_ERR_SHAPE), (dict(flags=4), tpg.MOE_ERR_UNSUPPORTED),
    (dict(flags=3), tpg.MOE_ERR_UNSUPPORTED), (dict(flags=-1), tpg.MOE_ERR_UNSUPPORTED),
])
def test_bad_problems_are_rejected_by_every_entry_point(kw, status):
    lib = tpg.load()
    p = ctypes.byref(_p(**kw))
    w = ctypes.byref(tpg.Weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    assert lib.moe_route_topk(FAKE, None, p, FAKE, FAKE, None) == status
    assert lib.moe_permute(FAKE, FAKE, FAKE, p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == status
    ev = (ctypes.c_void_p * tpg.MOE_N_PERMUTE_EVENTS)(*[FAKE] * tpg.MOE_N_PERMUTE_EVENTS)
    assert lib.moe_permute_timed(FAKE, FAKE, FAKE, p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None,
                                 ev) == status
    assert lib.moe_grouped_ffn(FAKE, FAKE, FAKE, w, p, FAKE, FAKE, 1 << 40, None) == status
    assert lib.moe_unpermute_combine(FAKE, FAKE, FAKE, p, FAKE, None) == status
    assert lib.moe_forward(FAKE, None, FAKE, FAKE, w, p, FAKE, FAKE, 1 << 40, None) == status
    assert lib.moe_forward_noalloc(FAKE, None, FAKE, FAKE, w, p, FAKE, None) == status
    assert lib.moe_workspace_bytes(p) == 0
    assert lib.moe_call_workspace_bytes(p, tpg.MOE_WS_PERMUTE) == 0


def test_null_pointers_are_rejected():
    lib = tpg.load()
    p = ctypes.byref(_p())
    w = ctypes.byref(tpg.Weights(FAKE, None, None, FAKE, None, None))
    NULL = tpg.MOE_ERR_NULL
    assert lib.moe_route_topk(None, None, p, FAKE, FAKE, None) == NULL
    assert lib.moe_route_topk(FAKE, None, p, None, FAKE, None) == NULL
    assert lib.moe_route_topk(FAKE, None, None, FAKE, FAKE, None) == NULL
    assert lib.moe_permute(FAKE, None, FAKE, p, FAKE, FAKE, None, FAKE, None, FAKE, 1 << 40, None) == NULL
    assert lib.moe_grouped_ffn(FAKE, None, FAKE, None, p, FAKE, FAKE, 1 << 40, None) == NULL
    assert lib.moe_grouped_ffn(None, None, FAKE, w, p, FAKE, FAKE, 1 << 40, None) == NULL
    assert lib.moe_unpermute_combine(FAKE, FAKE, None, p, FAKE, None) == NULL
    assert lib.moe_forward(FAKE, None, None, None, w, p, FAKE, FAKE, 1 << 40, None) == NULL
    assert lib.moe_w4a8_dequant_table(None, None) == NULL
    ev = (ctypes.c_void_p * tpg.MOE_N_PERMUTE_EVENTS)(FAKE, None, FAKE)
    assert lib.moe_permute_timed(FAKE, None, FAKE, p, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None, ev) == NULL
    assert lib.moe_permute_timed(FAKE, None, FAKE, p, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None,
                                 None) == NULL
    # W4A8 (NVFP4 or MXFP4 weights) needs the scale arrays too
    for prec in (tpg.MOE_PREC_W4A8, tpg.MOE_PREC_W4A8_MX):
        p4 = ctypes.byref(_p(prec=prec, H=256))
        assert lib.moe_forward(FAKE, None, FAKE, FAKE, w, p4, FAKE, FAKE, 1 << 40, None) == NULL
        assert lib.moe_forward(FAKE, None, FAKE, None, ctypes.byref(tpg.Weights(*[FAKE] * 6)), p4, FAKE, FAKE,
                               1 << 40, None) == NULL


def test_small_workspace_is_rejected():
    lib = tpg.load()
    pr = _p()
    p = ctypes.byref(pr)
    w = ctypes.byref(tpg.Weights(FAKE, None, None, FAKE, None, None))
    for which, call in [
        (tpg.MOE_WS_PERMUTE, lambda n: lib.moe_permute(FAKE, None, FAKE, p, FAKE, FAKE, FAKE, FAKE, None, FAKE, n,
                                                       None)),
        (tpg.MOE_WS_PERMUTE, lambda n: lib.moe_permute_timed(
            FAKE, None, FAKE, p, FAKE, FAKE, FAKE, FAKE, None, FAKE, n, None,
            (ctypes.c_void_p * tpg.MOE_N_PERMUTE_EVENTS)(*[FAKE] * tpg.MOE_N_PERMUTE_EVENTS))),
        (tpg.MOE_WS_GROUPED_FFN, lambda n: lib.moe_grouped_ffn(FAKE, None, FAKE, w, p, FAKE, FAKE, n, None)),
        (tpg.MOE_WS_FORWARD, lambda n: lib.moe_forward(FAKE, None, FAKE, None, w, p, FAKE, FAKE, n, None)),
    ]:
        need = tpg.moe_call_workspace_bytes(pr, which)
        assert need > 0
        assert call(need - 1) == tpg.MOE_ERR_WORKSPACE


def test_zero_tokens_returns_ok_without_touching_anything():
    lib = tpg.load()
    p = ctypes.byref(_p(T=0))
    w = ctypes.byref(tpg.Weights(None, None, None, None, None, None))
    assert lib.moe_route_topk(None, None, p, None, None, None) == tpg.MOE_OK
    assert lib.moe_permute(None, None, None, p, None, None, None, None, None, None, 0, None) == tpg.MOE_OK
    assert lib.moe_grouped_ffn(None, None, None, w, p, None, None, 0, None) == tpg.MOE_OK
    assert lib.moe_unpermute_combine(None, None, None, p, None, None) == tpg.MOE_OK
    assert lib.moe_forward(None, None, None, None, w, p, None, None, 0, None) == tpg.MOE_OK


def test_w4a8_tile_weights_argument_checks():
    lib = tpg.load()
    A, B, C, D = 1 << 20, 2 << 20, 3 << 20, 4 << 20  # disjoint fake device ranges (never touched)
    ok_shape = (2, 64, 512)
    assert lib.moe_w4a8_tile_weights(None, B, C, D, *ok_shape, tpg.MOE_PREC_W4A8, None) == tpg.MOE_ERR_NULL
    assert lib.moe_w4a8_tile_weights(A, B, C, None, *ok_shape, tpg.MOE_PREC_W4A8, None) == tpg.MOE_ERR_NULL
    assert lib.moe_w4a8_tile_weights(A, B, C, D, *ok_shape, tpg.MOE_PREC_BF16, None) == tpg.MOE_ERR_UNSUPPORTED
    for E, N, K in ((0, 64, 512), (2, 48, 512), (2, 64, 384), (2, 64, 128)):
        assert lib.moe_w4a8_tile_weights(A, B, C, D, E, N, K, tpg.MOE_PREC_W4A8_MX, None) == tpg.MOE_ERR_SHAPE
    # outputs overlapping the inputs (2 * 64 * 256 = 32 KB of codes from A)
    assert lib.moe_w4a8_tile_weights(A, B, A + 4096, D, *ok_shape, tpg.MOE_PREC_W4A8, None) == tpg.MOE_ERR_UNSUPPORTED
    assert lib.moe_w4a8_tile_weights(A, B, C, B, *ok_shape, tpg.MOE_PREC_W4A8, None) == tpg.MOE_ERR_UNSUPPORTED


def test_unknown_weight_layout_is_rejected():
    lib = tpg.load()
    for prec in (tpg.MOE_PREC_W4A8, tpg.MOE_PREC_W4A8_MX):
        p = ctypes.byref(_p(prec=prec, H=256))
        w = tpg.Weights(*[FAKE] * 6, 7)
        assert lib.moe_forward(FAKE, None, FAKE, FAKE, ctypes.byref(w), p, FAKE, FAKE, 1 << 40,
                               None) == tpg.MOE_ERR_UNSUPPORTED
        assert lib.moe_grouped_ffn(FAKE, FAKE, FAKE, ctypes.byref(w), p, FAKE, FAKE, 1 << 40,
                                   None) == tpg.MOE_ERR_UNSUPPORTED


def test_k_up_to_e_is_accepted():
    """1 <= k <= E <= 256: a problem with k above 32 passes the host checks (here it stops at the
    first NULL pointer) and gets a workspace"""
    lib = tpg.load()
    for E, k in ((64, 64), (256, 33), (256, 256)):
        pr = _p(E=E, k=k)
        assert tpg.moe_workspace_bytes(pr) > 0
        assert lib.moe_route_topk(None, None, ctypes.byref(pr), FAKE, FAKE, None) == tpg.MOE_ERR_NULL


def test_workspace_sizes():
    big = _p(T=32768, H=7168, I=2048, E=32, k=8, glu_interleave=32)
    n = tpg.moe_workspace_bytes(big)
    assert n == tpg.moe_call_workspace_bytes(big, tpg.MOE_WS_FORWARD)
    S = 32768 * 8
    # the bf16 forward gathers inside GEMM1 (T*H*2 < 2^31): it holds y_perm (bf16 [S][H]) and
    # h (bf16 [S][I]) but no x_perm; sized by shape only
    assert S * (7168 * 2 + 2048 * 2) <= n < S * (7168 * 2 * 2 + 2048 * 2)
    # too many token rows for 31-bit offsets into x: the forward runs the separate gather
    unfused = _p(T=131072, H=8192, I=1024, E=8, k=2)
    assert tpg.moe_workspace_bytes(unfused) >= 131072 * 2 * (8192 * 2 * 2 + 1024 * 2)
    # W4A8 gathers inside GEMM1 too: y_perm (bf16) and h (fp32, fp8 and scales) but no fp8 x_perm
    w4 = _p(T=256, H=7168, I=2048, E=32, k=8, prec=tpg.MOE_PREC_W4A8, swiglu_clamp=10.0)
    S4 = 256 * 8
    n4 = tpg.moe_workspace_bytes(w4)
    assert S4 * (7168 * 2 + 2048 * 5) <= n4 < S4 * (7168 * 2 + 2048 * 5 + 7168)
    # MXFP4 weights change only the weight scales: the same workspace for every call
    mx = _p(T=256, H=7168, I=2048, E=32, k=8, prec=tpg.MOE_PREC_W4A8_MX, swiglu_clamp=10.0)
    for which in (tpg.MOE_WS_PERMUTE, tpg.MOE_WS_GROUPED_FFN, tpg.MOE_WS_FORWARD):
        assert tpg.moe_call_workspace_bytes(mx, which) == tpg.moe_call_workspace_bytes(w4, which) > 0
    assert (tpg.moe_call_workspace_bytes(big, tpg.MOE_WS_PERMUTE)
            < tpg.moe_call_workspace_bytes(big, tpg.MOE_WS_GROUPED_FFN) < n)
    assert tpg.moe_call_workspace_bytes(big, 99) == 0


def test_single_launch_flag_needs_an_eligible_problem():
    """MOE_FLAG_SINGLE_LAUNCH: W4A8 only, at most 256 tokens and 2048 slots, H and I multiples of 1024;
    otherwise MOE_ERR_UNSUPPORTED before anything is enqueued"""
    lib = tpg.load()
    w = ctypes.byref(tpg.Weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    one = tpg.MOE_FLAG_SINGLE_LAUNCH
    for kw in (dict(prec=0, H=1024, I=1024), dict(prec=1, T=300, H=1024, I=1024),
               dict(prec=2, T=256, k=16, E=32, H=1024, I=1024), dict(prec=1, H=1536, I=1024),
               dict(prec=2, H=1024, I=512)):
        pr = _p(flags=one, **kw)
        n = tpg.moe_workspace_bytes(pr)
        assert n > 0
        assert lib.moe_forward(FAKE, None, FAKE, FAKE, w, ctypes.byref(pr), FAKE, FAKE, n, None) == \
            tpg.MOE_ERR_UNSUPPORTED, kw


def test_scatter_flag_is_accepted_alone_by_every_precision():
    """MOE_FLAG_SCATTER_Y passes the problem check for every precision (the workspace is sized the
    same); with MOE_FLAG_SINGLE_LAUNCH beside it the problem is refused"""
    for prec in (tpg.MOE_PREC_BF16, tpg.MOE_PREC_W4A8, tpg.MOE_PREC_W4A8_MX):
        plain = _p(prec=prec, H=1024, I=1024)
        scat = _p(prec=prec, H=1024, I=1024, flags=tpg.MOE_FLAG_SCATTER_Y)
        assert tpg.moe_workspace_bytes(scat) == tpg.moe_workspace_bytes(plain) > 0
        both = _p(prec=prec, H=1024, I=1024, flags=tpg.MOE_FLAG_SCATTER_Y | tpg.MOE_FLAG_SINGLE_LAUNCH)
        assert tpg.moe_workspace_bytes(both) == 0


def test_noalloc_refuses_problems_beyond_its_scratch_on_the_host():
    """the check comes before any HIP call (no device is touched here)"""
    lib = tpg.load()
    w = ctypes.byref(tpg.Weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE))
    big = _p(T=4096, H=7168, I=2048, E=32, k=8)
    assert tpg.moe_workspace_bytes(big) > tpg.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(FAKE, None, FAKE, None, w, ctypes.byref(big), FAKE, None) == tpg.MOE_ERR_SCRATCH
    assert b"64 MiB" in lib.moe_status_str(tpg.MOE_ERR_SCRATCH)
    # the W4A8 decode layer up to 256 tokens fits
    dec = _p(T=256, H=7168, I=2048, E=32, k=8, prec=tpg.MOE_PREC_W4A8_MX, swiglu_clamp=10.0)
    assert tpg.moe_workspace_bytes(dec) <= tpg.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(FAKE, None, FAKE, FAKE, w, ctypes.byref(_p(T=0)), FAKE, None) == tpg.MOE_OK


def test_status_strings():
    lib = tpg.load()
    for s in range(7):
        assert lib.moe_status_str(s)
    assert lib.moe_status_str(42) == b"unknown status"
