"""The seeded input generator: determinism, structure, bf16 rounding."""
import numpy as np
import pytest

import synth
from synth import CONFIGS, IGNORE_INDEX, make_case


def test_deterministic_and_block_invariant():
    cfg = synth.small_config("c2", N=64, H=48, V=300)
    a = make_case(cfg)
    b = make_case(cfg)
    assert a.digest() == b.digest()
    # drawing W in row blocks gives the same values as one draw
    rng = np.random.default_rng(cfg.seed)
    rng.standard_normal((64, 48), dtype=np.float32)
    W_once = rng.standard_normal((300, 48), dtype=np.float32) * np.float32(0.02)
    assert np.array_equal(a.W, synth.f32_to_bf16_bits(W_once))
    rng2 = np.random.default_rng(cfg.seed)
    h2 = synth._draw_matrix(rng2, 64, 48, 1.0, "bf16", block_rows=7)
    W2 = synth._draw_matrix(rng2, 300, 48, 0.02, "bf16", block_rows=13)
    assert np.array_equal(h2, a.h) and np.array_equal(W2, a.W)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_ignore_counts(name):
    cfg = CONFIGS[name]
    case = make_case(cfg, H=8, V=cfg.V if cfg.V < 5000 else 5000)
    n_ign = int(np.sum(case.labels == IGNORE_INDEX))
    assert n_ign == int(round(cfg.ignore_frac * cfg.N))
    valid = case.labels != IGNORE_INDEX
    assert np.all((case.labels[valid] >= 0) & (case.labels[valid] < case.cfg.V))


def test_valid_row_counts_of_the_workloads():
    assert [CONFIGS[k].n_valid for k in ("c1", "c2", "c3", "c4", "c5")] == [230, 3891, 7782, 7782, 26214]


def test_tail_padding_runs():
    cfg = CONFIGS["c5"]
    case = make_case(cfg, H=8, V=1000)
    lab = case.labels.reshape(4, 8192)
    runs = []
    for s in range(4):
        ign = lab[s] == IGNORE_INDEX
        L = int(ign.sum())
        runs.append(L)
        assert np.all(ign[8192 - L:]) and not np.any(ign[:8192 - L])
    assert runs == [1638, 1638, 1639, 1639]


def test_zipf_shape():
    rng = np.random.default_rng(0)
    V = 1000
    x = synth.zipf_labels(rng, 200000, V, 1.1)
    assert x.min() >= 0 and x.max() < V
    k = np.arange(1, V + 1, dtype=np.float64)
    p = k ** -1.1
    p /= p.sum()
    counts = np.bincount(x, minlength=V)
    # the three most frequent ids carry the law's mass within sampling noise
    for t in range(3):
        assert abs(counts[t] / 200000 - p[t]) < 5 * np.sqrt(p[t] / 200000)
    assert counts[0] > counts[1] > counts[2]


def test_bf16_round_to_nearest_even_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32)
    # include exact ties: low 16 bits == 0x8000
    ties = (rng.integers(0, 2**16, 64).astype(np.uint32) << 16) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)[np.isfinite(ties.view(np.float32))]])
    ours = synth.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
