"""Host replay of the index arithmetic of the W4A8 GEMMs, the single-launch small-token forward and
the two small front ends (tests/replay/w4a8_replay.cpp, built with g++ from the kernels' own index
functions in w4a8_index.h): every buffer load inside its descriptor or wholly beyond it, no 32-bit
offset wrapping, every LDS access inside its array, every store inside its buffer, for the decode
layer at every token count, the small GPU cases, random shapes up to E = 256, k = 32, 2048 slots, and
the W4A8 problems of the GPU forward sweep (tests/_sweep.py)."""
import os
import subprocess

import pytest

from tests._sweep import N_CASES, draw

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_w4a8_index_replay(tmp_path):
    exe = str(tmp_path / "w4a8_replay")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-o", exe,
                    os.path.join(HERE, "replay", "w4a8_replay.cpp")], check=True)
    extra = tmp_path / "sweep_problems.txt"
    with open(extra, "w") as f:
        for i in range(N_CASES):
            cfg, _ = draw(i)
            if cfg.prec != "bf16":
                f.write(f"{cfg.T} {cfg.H} {cfg.I} {cfg.E} {cfg.k}\n")
    r = subprocess.run([exe, str(extra)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:]
    assert " 0 out of range" in r.stdout
