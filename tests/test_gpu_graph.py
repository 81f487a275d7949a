"""moe_forward captured in a HIP graph (through torch.cuda.CUDAGraph).

The entry points allocate nothing and never synchronise, and the workspace size is a
function of the problem alone (FlashInfer "[SM90] Add W4A8 MegaMoE support": buffers
are allocated by the caller before graph capture), so one capture must serve every
later call of the same shape.  Between replays the test rewrites the captured input
buffers with a second seed's logits and activations (another routing: different
counts, offsets and GEMM tile lists, all built on the device) and runs eager work and
synchronisations; every replay must equal the eager forward of its inputs bitwise.
"""
from __future__ import annotations

import pytest
import torch

import token_permute_grouped_amd as tpg
from moe_synth import MoeConfig, generate
from tests._gpu import DEV, DeviceProblem, bf16_host

pytestmark = pytest.mark.gpu

CASES = [
    MoeConfig("graph_bf16", T=200, H=256, I=384, E=16, k=4),
    MoeConfig("graph_bf16_il_drop", T=300, H=512, I=256, E=8, k=3, glu_interleave=32, drop_p=0.1),
    MoeConfig("graph_w4a8", T=64, H=512, I=256, E=8, k=2, prec="w4a8", swiglu_clamp=10.0),
    # K a multiple of 1024 and T <= 32: the persistent W4A8 GEMMs
    MoeConfig("graph_w4a8_persistent", T=16, H=1024, I=1024, E=32, k=8, prec="w4a8", swiglu_clamp=10.0),
    MoeConfig("graph_w4a8_mx_persistent", T=16, H=1024, I=1024, E=32, k=8, prec="w4a8_mx", swiglu_clamp=10.0),
    MoeConfig("graph_w4a8_mx", T=64, H=512, I=256, E=8, k=2, prec="w4a8_mx", swiglu_clamp=10.0),
    # one token: GEMM1 split in two K halves (partial sums added by the re-quantisation), both formats
    MoeConfig("graph_w4a8_t1_split", T=1, H=1024, I=1024, E=8, k=4, prec="w4a8", swiglu_clamp=10.0),
    MoeConfig("graph_w4a8_mx_t1_split", T=1, H=1024, I=1024, E=8, k=4, prec="w4a8_mx", swiglu_clamp=10.0),
    # three-block (merged) m-tiles: every expert holds 65..85 rows
    MoeConfig("graph_w4a8_merged", T=200, H=512, I=512, E=5, k=2, prec="w4a8", glu_interleave=32, swiglu_clamp=10.0,
              drop_p=0.05),
    # the single-launch forward with two token blocks per tile (its hand-off words reset in-kernel)
    MoeConfig("graph_w4a8_mx_fused_t100", T=100, H=1024, I=1024, E=16, k=4, prec="w4a8_mx", glu_interleave=32,
              swiglu_clamp=10.0, drop_p=0.1),
]


def _eager(d: DeviceProblem):
    return bf16_host(d.forward())


SINGLE = {"graph_w4a8_persistent", "graph_w4a8_mx_fused_t100", "graph_w4a8_t1_split", "graph_w4a8_mx_t1_split"}  # also with MOE_FLAG_SINGLE_LAUNCH


SCATTER = {"graph_bf16_il_drop", "graph_w4a8_persistent", "graph_w4a8_merged"}  # also with MOE_FLAG_SCATTER_Y
FLAG_IDS = {0: "default", tpg.MOE_FLAG_SINGLE_LAUNCH: "single_launch", tpg.MOE_FLAG_SCATTER_Y: "scatter_y"}


@pytest.mark.parametrize("cfg,flags", [(c, 0) for c in CASES]
                         + [(c, tpg.MOE_FLAG_SINGLE_LAUNCH) for c in CASES if c.name in SINGLE]
                         + [(c, tpg.MOE_FLAG_SCATTER_Y) for c in CASES if c.name in SCATTER],
                         ids=lambda v: v.name if isinstance(v, MoeConfig) else FLAG_IDS[v])
def test_forward_graph_replay(cfg, flags):
    print(f"[gpu graph] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} {cfg.prec} flags={flags}",
          flush=True)
    inp_a, other = generate(cfg, seed=0), generate(cfg, seed=1)
    # the second input set: seed 1's logits, activations (and drop mask) with seed 0's weights
    inp_b = dict(inp_a, **{k: other[k] for k in ("logits", "x", "x_scale", "slot_drop") if k in other})
    da, db = DeviceProblem(inp_a, flags), DeviceProblem(inp_b, flags)
    want = [_eager(da), _eager(db)]
    assert (want[0] != want[1]).any()  # the two routings differ

    # the captured call's own buffers (the weights are shared: only the inputs change)
    logits, x = da.logits.clone(), da.x.clone()
    x_scale = da.x_scale.clone() if da.x_scale is not None else None
    drop = da.drop.clone() if da.drop is not None else None
    ws = da.workspace(tpg.MOE_WS_FORWARD, fill=0x5A)
    out = torch.full((cfg.T, cfg.H), -1, dtype=torch.int16, device=DEV)

    def call():
        tpg.moe_forward(logits, drop, x, x_scale, da.weights, da.p, out, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for i in range(6):
        src = da if i % 2 == 0 else db
        logits.copy_(src.logits)
        x.copy_(src.x)
        if x_scale is not None:
            x_scale.copy_(src.x_scale)
        if drop is not None:
            drop.copy_(src.drop)
        out.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bf16_host(out)
        n_diff = int((got != want[i % 2]).sum())
        print(f"[gpu graph] {cfg.name}: replay {i} (seed {i % 2}): {n_diff} differing elements", flush=True)
        assert n_diff == 0
        # eager work between replays, on the same stream
        _ = _eager(db if i % 2 == 0 else da)
