"""Seeded random problems for the forward sweep (tests/test_gpu_shape_sweep.py) and the host index
replay of the same shapes (tests/test_index_replay.py).  Shapes come from the ranges the library
accepts: H and I multiples of 128 (of 256 for the W4A8 precisions), 1 <= k <= E <= 256."""
from __future__ import annotations

import numpy as np

from moe_synth import MoeConfig

N_CASES = 48


def draw(i: int) -> tuple[MoeConfig, bool]:
    """case i (16 per precision): the problem and whether the forward takes the scatter epilogue"""
    rng = np.random.default_rng(9000 + i)
    prec = ("bf16", "w4a8", "w4a8_mx")[i % 3]
    gran = 128 if prec == "bf16" else 256
    E = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    H = gran * int(rng.integers(1, 5))
    I = gran * int(rng.integers(1, 5))
    while E * H * I > (1 << 25) and max(H, I) > gran:  # keep the weights a few hundred MB at most
        if H >= I:
            H -= gran
        else:
            I -= gran
    T = int(rng.choice([1, 2, 7, 31, 32, 33, 64, 100, 257, 600]))
    cfg = MoeConfig(f"sweep{i}_{prec}", T=T, H=H, I=I, E=E, k=k, prec=prec,
                    glu_interleave=int(rng.choice([0, 32])),
                    swiglu_clamp=float(rng.choice([0.0, 0.5, 10.0])),
                    zipf_s=float(rng.choice([0.0, 1.2])),
                    drop_p=float(rng.choice([0.0, 0.1])))
    return cfg, bool(rng.random() < 0.5)
