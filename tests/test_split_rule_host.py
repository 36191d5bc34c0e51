"""CPU test of the chunk planner's grad_h split rule (``grad_h_split``),
built for the host with g++: against a plain model of the rule written with
exact fractions, over the page shapes and a grid of tile and K-step counts.

The rule: among splits s <= s_max of the vocabulary's K steps that leave at
least 64 steps per split (or s = 1), the best wave efficiency over 256 CUs
(split tiles / (waves * 256)); among equally efficient ones, the smallest s
with at least 12 waves of tiles still >= 256 K steps long, else the smallest.
"""
import os
import shutil
import subprocess
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_gemm_amd", "csrc")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ and the ROCm headers are needed")
    exe = str(tmp_path_factory.mktemp("split") / "split_host")
    subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(ROOT, "tests", "host", "split_host.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def run(exe, triples):
    inp = "".join(f"{t} {k} {s}\n" for t, k, s in triples)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split()
    return [(int(out[2 * i]), int(out[2 * i + 1])) for i in range(len(triples))]


def model(tiles, ksteps, s_max):
    cands = [s for s in range(1, min(s_max, 16) + 1) if s == 1 or ksteps // s >= 64]
    stats = {}
    for s in cands:
        per = -(-ksteps // s)
        real = -(-ksteps // per)
        waves = -(-(tiles * real) // 256)
        stats[s] = (Fraction(tiles * real, waves * 256) if waves else Fraction(0), waves, real, per)
    best = max(e for e, _, _, _ in stats.values())
    good = [s for s in cands if stats[s][0] == best]
    long_enough = [s for s in good if stats[s][1] >= 12 and ksteps // stats[s][2] >= 256]
    s = (long_enough or good)[0]
    return stats[s][2], stats[s][3]


def test_page_shapes(harness):
    cases = [
        (416, 3160, 16),   # c4 chunk (16 x 26 tiles, V padded to 202240): 8 splits, 13 waves
        (448, 2020, 16),   # c3 chunk (16 x 28): 4 splits
        (1792, 2020, 16),  # c5 chunk (64 x 28): 2 splits
        (128, 2004, 16),   # c2 chunk (8 x 16, V padded to 128256): 2 splits
        (390, 3160, 8),    # 15 token tiles and at most 8 splits: 7 splits, 11 waves
        (0, 3160, 8),      # no tiles
    ]
    got = run(harness, cases)
    assert got == [model(*c) for c in cases]
    assert [g[0] for g in got] == [8, 4, 2, 2, 7, 1]


def test_rule_matches_the_model_on_a_grid(harness):
    cases = [(t, k, s) for t in (1, 2, 7, 16, 26, 100, 255, 256, 257, 390, 416, 1000, 4097)
             for k in (1, 4, 63, 64, 127, 128, 500, 2020, 3160, 10000)
             for s in (1, 2, 3, 5, 8, 16, 40)]
    got = run(harness, cases)
    for c, g in zip(cases, got):
        assert g == model(*c), c
        splits, per = g
        t, k, s = c
        # the splits cover the K steps exactly once and never exceed the cap
        assert 1 <= splits <= max(1, min(s, 16)) and (splits - 1) * per < k <= splits * per
