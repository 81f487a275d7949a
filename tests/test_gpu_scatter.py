"""GPU: the scatter epilogue (MOE_FLAG_SCATTER_Y).  GEMM2 stores every output row at its slot
t*k + j and the combine reads a token's k rows in slot order; the forward must be bitwise the
default forward's (the same rows, summed in the same order), for every precision, GEMM form
(one tile per workgroup, the persistent W4A8 form, the K-split W4A8 GEMM1) and with dropped
slots, whose rows nobody writes (the workspace fill would show in the output if the combine
read one)."""
from __future__ import annotations

import pytest

import token_permute_grouped_amd as tpg
from moe_synth import CONFIGS, MoeConfig, generate
from tests._gpu import DeviceProblem, bf16_host

pytestmark = pytest.mark.gpu

CASES = [
    CONFIGS["tiny"],
    MoeConfig("sc_one_token", T=1, H=256, I=384, E=4, k=4),
    MoeConfig("sc_ragged_drop", T=700, H=256, I=640, E=5, k=2, drop_p=0.1),
    MoeConfig("sc_h_odd_tile", T=300, H=384, I=256, E=8, k=3, glu_interleave=32, swiglu_clamp=1.0),
    MoeConfig("sc_wide_k", T=40, H=128, I=128, E=128, k=64),
    CONFIGS["mid"],
    CONFIGS["skewed"],
    # W4A8: T <= 32 with K a multiple of 1024 runs the persistent GEMMs, one token with NVFP4 the
    # K-split GEMM1; merged three-block tiles; both weight formats
    MoeConfig("sc_w4_one_token_split", T=1, H=1024, I=512, E=8, k=4, prec="w4a8", swiglu_clamp=10.0),
    MoeConfig("sc_w4_persistent_drop", T=32, H=1024, I=1024, E=64, k=8, prec="w4a8", glu_interleave=32,
              swiglu_clamp=10.0, drop_p=0.1),
    MoeConfig("sc_w4_merged_drop", T=200, H=512, I=512, E=5, k=2, prec="w4a8", swiglu_clamp=10.0, drop_p=0.05),
    MoeConfig("sc_mx_persistent", T=16, H=1024, I=1024, E=32, k=8, prec="w4a8_mx", swiglu_clamp=10.0),
    MoeConfig("sc_mx_ragged_drop", T=300, H=768, I=768, E=5, k=2, prec="w4a8_mx", drop_p=0.1),
    CONFIGS["w4a8"],
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_scatter_forward_equals_default(cfg):
    print(f"[gpu scatter] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} {cfg.prec}", flush=True)
    d = DeviceProblem(generate(cfg, seed=3))
    ref = bf16_host(d.forward())
    d.p.flags = tpg.MOE_FLAG_SCATTER_Y  # the same resident inputs and weights
    # two calls on one workspace: the second sees the first's y rows, the first only the fill
    ws = d.workspace(tpg.MOE_WS_FORWARD, fill=0xEF)
    outs = [bf16_host(d.forward(ws)) for _ in range(2)]
    n_diff = [int((o != ref).sum()) for o in outs]
    print(f"[gpu scatter] {cfg.name}: differing elements {n_diff}", flush=True)
    assert n_diff == [0, 0]
