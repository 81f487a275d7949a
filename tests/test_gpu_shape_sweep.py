"""GPU: the whole forward on seeded random problems against the oracle.

Each case draws its shape from the ranges the library accepts (H and I multiples of 128, of 256
for the W4A8 precisions; 1 <= k <= E <= 256) together with a ragged token count, Zipf-skewed or
uniform routing, dropped slots, the SwiGLU clamp, the interleaved W1 layout and the default or
scatter-epilogue forward, so the drawn problems land on every GEMM form (one tile per workgroup,
the persistent W4A8 GEMMs at T <= 32 with K a multiple of 1024, the K-split GEMM1 at decode
sizes, merged last tiles) and on both front ends.  Every token is compared; the bars are the
per-precision ones of the other parity tests (max|err| / max|ref| <= 2e-2 for bf16, 3e-2 for
W4A8), and every output row must be written.  The W4A8 shapes also go through the host index replay."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import token_permute_grouped_amd as tpg
from moe_synth import generate
from tests._gpu import DeviceProblem, assert_all_rows_written, bf16_f64, bf16_host, rel_err, to_dev
from tests._sweep import N_CASES, draw

pytestmark = pytest.mark.gpu

BARS = {"bf16": 2e-2, "w4a8": 3e-2, "w4a8_mx": 3e-2}


@pytest.mark.parametrize("i", range(N_CASES))
def test_forward_on_a_drawn_problem(i):
    cfg, scatter = draw(i)
    flags = tpg.MOE_FLAG_SCATTER_Y if scatter else 0
    print(f"[gpu sweep] case {i}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} {cfg.prec} "
          f"il={cfg.glu_interleave} clamp={cfg.swiglu_clamp} zipf={cfg.zipf_s} drop={cfg.drop_p} flags={flags}",
          flush=True)
    inp = generate(cfg, seed=i)
    d = DeviceProblem(inp, flags=flags)
    out = bf16_host(d.forward())
    ref = oracle.moe_forward(inp)
    err = rel_err(bf16_f64(out), ref)
    print(f"[gpu sweep] case {i}: max|err|/max|ref| = {err:.3e}", flush=True)
    assert err <= BARS[cfg.prec]
    assert_all_rows_written(to_dev(out), cfg.T, float(np.abs(ref).max()), cfg.name)
