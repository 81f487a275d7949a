"""moe_forward_noalloc (the entry point for callers that cannot allocate) against moe_forward.

Both run the same kernels on the same inputs, the no-allocation one on the library's own
device scratch instead of a caller's workspace, so the outputs must be bitwise equal.  The
calls come in a row with shrinking inputs (the scratch keeps the previous call's contents),
in both precisions, and one problem too large for the scratch is refused on the host."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import token_permute_grouped_amd as tpg
from moe_synth import CONFIGS, MoeConfig, generate
from tests._gpu import DEV, DeviceProblem, bf16_f64, bf16_host, rel_err

pytestmark = pytest.mark.gpu

CASES = [
    MoeConfig("na_ragged", T=700, H=256, I=640, E=5, k=2),
    MoeConfig("na_tiny", T=64, H=128, I=256, E=8, k=2),
    CONFIGS["w4a8_mx"].with_tokens(64),
    CONFIGS["w4a8_mx"].with_tokens(8),
    MoeConfig("na_w4_drop", T=30, H=512, I=512, E=6, k=3, prec="w4a8", glu_interleave=32, swiglu_clamp=10.0,
              drop_p=0.1),
    CONFIGS["w4a8"].with_tokens(4),  # also run with MOE_FLAG_SINGLE_LAUNCH below
]
# flags of call i (the scatter epilogue on two calls, the single launch on the last)
FLAGS = {1: tpg.MOE_FLAG_SCATTER_Y, 4: tpg.MOE_FLAG_SCATTER_Y, len(CASES) - 1: tpg.MOE_FLAG_SINGLE_LAUNCH}


def _noalloc(d: DeviceProblem):
    cfg = d.cfg
    out = torch.full((cfg.T, cfg.H), -1, dtype=torch.int16, device=DEV)
    tpg.moe_forward_noalloc(d.logits, d.drop, d.x, d.x_scale, d.weights, d.p, out)
    return out


def test_noalloc_forward_equals_forward_on_calls_in_a_row():
    for i, cfg in enumerate(CASES):
        print(f"[no-alloc] call {i}: {cfg.name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} {cfg.prec} "
              f"flags={FLAGS.get(i, 0)}", flush=True)
        inp = generate(cfg, seed=i)
        d = DeviceProblem(inp, FLAGS.get(i, 0))
        assert tpg.moe_workspace_bytes(d.p) <= tpg.MOE_NOALLOC_SCRATCH_BYTES
        a = bf16_host(_noalloc(d))
        b = bf16_host(d.forward())
        n_diff = int((a != b).sum())
        assert n_diff == 0, f"{cfg.name}: {n_diff} elements differ from moe_forward"
        tokens = np.arange(min(cfg.T, 16))
        err = rel_err(bf16_f64(a[tokens]), oracle.moe_forward(inp, tokens))
        assert err <= (2e-2 if cfg.prec == "bf16" else 3e-2), (cfg.name, err)
        del d


def test_noalloc_refuses_a_problem_larger_than_its_scratch():
    p = tpg.make_problem(256, 7168, 2048, 32, 32, tpg.MOE_PREC_BF16)
    assert tpg.moe_workspace_bytes(p) > tpg.MOE_NOALLOC_SCRATCH_BYTES
    t = torch.zeros(4, dtype=torch.int16, device=DEV)
    w = tpg.make_weights(t, t)
    with pytest.raises(tpg.MoeError) as ei:
        tpg.moe_forward_noalloc(t, None, t, None, w, p, t)
    assert ei.value.status == tpg.MOE_ERR_SCRATCH
