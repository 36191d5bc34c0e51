"""Pins for the fp64 oracle (``oracle/``), independent of the oracle itself.

Each check is chosen so that a plausible mistake in the oracle (a dropped
term, a wrong sign or index, a transposed operand, the multiplier on the wrong
side of the cap, the wrong mean denominator) fails at least one of them:

* closed forms: W = 0 gives loss ln V and a closed-form grad_W; a hand-worked
  two-class case with tanh(ln 3) = 0.8;
* invariants: rows of d loss / d logits sum to 0; columns of grad_W sum to 0
  without a softcap; equal W rows give ln V and zero grad_h; ignored rows
  contribute nothing;
* the multiplier fold of the Muse Glimmer page (Details > Softcap):
  (m h) W^T = m (h W^T);
* T -> infinity recovers the uncapped loss;
* central finite differences on tiny shapes with a strongly nonlinear cap;
* torch's fp64 cross_entropy + autograd on the explicitly capped logits (an
  independent library implementation of the same composite);
* brute-force argmax with ties;
* per-row upstream gradients (reduction "none") and a scalar upstream
  gradient against torch's fp64 autograd with those upstream gradients, plus
  linearity in the row weights.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.flce import flce_reference, grad_h_rows, grad_W_rows, row_stats

IGN = -100


def _rand(N, H, V, seed=0, scale=0.5, n_ign=1):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H))
    W = scale * rng.standard_normal((V, H))
    labels = rng.integers(0, V, N)
    if n_ign:
        labels[rng.choice(N, n_ign, replace=False)] = IGN
    return h, W, labels


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("T,m", [(0.0, 1.0), (30.0, 0.5), (1.0, 0.37)])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_zero_weight_closed_form(T, m, reduction):
    N, H, V = 7, 5, 11
    rng = np.random.default_rng(1)
    h = rng.standard_normal((N, H))
    W = np.zeros((V, H))
    labels = rng.integers(0, V, N)
    labels[[1, 4]] = IGN
    valid = labels != IGN
    nv = int(valid.sum())
    r = flce_reference(h, W, labels, IGN, T, m, reduction)
    s = 1.0 / nv if reduction == "mean" else 1.0
    assert r["loss"] == pytest.approx(s * nv * math.log(V), rel=1e-14)
    assert np.all(r["grad_h"] == 0.0)
    # grad_W[v] = m s ((1/V) sum_valid h_i - sum_{valid, label_i = v} h_i)
    exp_gW = np.tile(h[valid].sum(0) / V, (V, 1))
    for i in np.nonzero(valid)[0]:
        exp_gW[labels[i]] -= h[i]
    exp_gW *= m * s
    np.testing.assert_allclose(r["grad_W"], exp_gW, rtol=1e-12, atol=1e-15)
    # all logits tie, the lowest index wins
    assert np.all(r["pred"] == 0)


def test_hand_worked_two_class():
    """h = [1], W = [[0], [ln 3]], label 0.
    No cap: softmax = (1/4, 3/4), loss = ln 4, d/da = (-3/4, 3/4),
    grad_h = (3/4) ln 3, grad_W = (-3/4, 3/4).
    Cap T = 1: z = (0, tanh(ln 3)) = (0, 0.8) exactly, loss = ln(1 + e^0.8),
    d/da_1 = p1 (1 - 0.8^2), d/da_0 = -p1 with p1 = e^0.8 / (1 + e^0.8)."""
    h = np.array([[1.0]])
    W = np.array([[0.0], [math.log(3.0)]])
    lab = np.array([0])
    r = flce_reference(h, W, lab, IGN, 0.0, 1.0, "mean")
    assert r["loss"] == pytest.approx(math.log(4.0), rel=1e-15)
    assert r["grad_h"][0, 0] == pytest.approx(0.75 * math.log(3.0), rel=1e-14)
    np.testing.assert_allclose(r["grad_W"][:, 0], [-0.75, 0.75], rtol=1e-14)
    assert r["n_correct"] == 0 and r["pred"][0] == 1

    r = flce_reference(h, W, lab, IGN, 1.0, 1.0, "mean")
    p1 = math.exp(0.8) / (1.0 + math.exp(0.8))
    assert r["loss"] == pytest.approx(math.log1p(math.exp(0.8)), rel=1e-14)
    np.testing.assert_allclose(r["z"][0], [0.0, 0.8], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(r["grad_W"][:, 0], [-p1, 0.36 * p1], rtol=1e-13)
    assert r["grad_h"][0, 0] == pytest.approx(0.36 * p1 * math.log(3.0), rel=1e-13)


def test_equal_weight_rows():
    N, H, V = 6, 4, 9
    rng = np.random.default_rng(2)
    h = rng.standard_normal((N, H))
    W = np.tile(rng.standard_normal(H), (V, 1))
    labels = rng.integers(0, V, N)
    for T in (0.0, 2.0):
        r = flce_reference(h, W, labels, IGN, T, 0.7, "mean")
        assert r["loss"] == pytest.approx(math.log(V), rel=1e-12)
        np.testing.assert_allclose(r["grad_h"], 0.0, atol=1e-13)


# ------------------------------------------------------------------ invariants

def test_dlogit_rows_sum_to_zero_and_grad_W_columns():
    h, W, labels = _rand(12, 6, 17, seed=3)
    r = flce_reference(h, W, labels, IGN, 0.0, 0.8, "mean")
    valid = labels != IGN
    np.testing.assert_allclose(r["dlogits"][valid].sum(1), 0.0, atol=1e-15)
    np.testing.assert_allclose(r["grad_W"].sum(0), 0.0, atol=1e-14)
    # with a cap, d loss / d z still sums to zero; d loss / d a does not
    rc = flce_reference(h, W, labels, IGN, 1.0, 0.8, "mean")
    dz = rc["dlogits"] / (1.0 - np.tanh(0.8 * (h @ W.T) / 1.0) ** 2)
    np.testing.assert_allclose(dz[valid].sum(1), 0.0, atol=1e-14)
    assert np.max(np.abs(rc["dlogits"][valid].sum(1))) > 1e-6


def test_ignored_rows():
    h, W, labels = _rand(10, 5, 13, seed=4, n_ign=3)
    ign = np.nonzero(labels == IGN)[0]
    r = flce_reference(h, W, labels, IGN, 1.5, 0.6, "mean")
    assert np.all(r["grad_h"][ign] == 0.0)
    assert np.all(r["loss_rows"][ign] == 0.0)
    h2 = h.copy()
    h2[ign] += 3.0
    r2 = flce_reference(h2, W, labels, IGN, 1.5, 0.6, "mean")
    assert r2["loss"] == pytest.approx(r["loss"], rel=1e-14)
    np.testing.assert_allclose(r2["grad_W"], r["grad_W"], rtol=1e-13, atol=1e-16)


def test_all_rows_ignored():
    h, W, labels = _rand(4, 3, 5, seed=5, n_ign=0)
    labels[:] = IGN
    for red in ("mean", "sum"):
        r = flce_reference(h, W, labels, IGN, 0.0, 1.0, red)
        assert r["loss"] == 0.0 and r["n_correct"] == 0
        assert np.all(r["grad_h"] == 0.0) and np.all(r["grad_W"] == 0.0)


def test_mean_is_sum_over_n_valid():
    h, W, labels = _rand(9, 4, 8, seed=6, n_ign=2)
    rm = flce_reference(h, W, labels, IGN, 2.0, 0.9, "mean")
    rs = flce_reference(h, W, labels, IGN, 2.0, 0.9, "sum")
    nv = int((labels != IGN).sum())
    assert rm["loss"] == pytest.approx(rs["loss"] / nv, rel=1e-14)
    np.testing.assert_allclose(rm["grad_W"], rs["grad_W"] / nv, rtol=1e-13, atol=1e-17)


def test_multiplier_fold():
    """(m h) W^T == m (h W^T): running with multiplier m equals running on
    m*h with multiplier 1; grad_h picks up the chain factor m."""
    h, W, labels = _rand(8, 6, 10, seed=7)
    m = 0.37
    for T in (0.0, 1.0):
        r1 = flce_reference(h, W, labels, IGN, T, m, "mean")
        r2 = flce_reference(m * h, W, labels, IGN, T, 1.0, "mean")
        assert r1["loss"] == pytest.approx(r2["loss"], rel=1e-13)
        np.testing.assert_allclose(r1["grad_W"], r2["grad_W"], rtol=1e-12, atol=1e-16)
        np.testing.assert_allclose(r1["grad_h"], m * r2["grad_h"], rtol=1e-12, atol=1e-16)


def test_multiplier_inside_the_cap():
    """The cap sees m * logits: T tanh(m a / T), not m T tanh(a / T)."""
    h, W, labels = _rand(3, 4, 6, seed=8, n_ign=0)
    m, T = 0.5, 0.7
    r = flce_reference(h, W, labels, IGN, T, m, "mean")
    np.testing.assert_allclose(r["z"], T * np.tanh(m * (h @ W.T) / T), rtol=1e-14)


def test_softcap_to_infinity_is_uncapped():
    h, W, labels = _rand(10, 6, 12, seed=9)
    r0 = flce_reference(h, W, labels, IGN, 0.0, 0.8, "mean")
    rinf = flce_reference(h, W, labels, IGN, 1e8, 0.8, "mean")
    assert rinf["loss"] == pytest.approx(r0["loss"], rel=1e-12)
    np.testing.assert_allclose(rinf["grad_h"], r0["grad_h"], rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(rinf["grad_W"], r0["grad_W"], rtol=1e-9, atol=1e-14)


# --------------------------------------------------------- finite differences

@pytest.mark.parametrize("reduction", ["mean", "sum"])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_central_finite_differences(reduction, T):
    N, H, V = 4, 3, 5
    h, W, labels = _rand(N, H, V, seed=10, scale=1.0, n_ign=1)
    m = 0.37

    def L(hh, WW):
        return flce_reference(hh, WW, labels, IGN, T, m, reduction)["loss"]

    r = flce_reference(h, W, labels, IGN, T, m, reduction)
    eps = 1e-6
    gh = np.zeros_like(h)
    for idx in np.ndindex(*h.shape):
        hp, hm = h.copy(), h.copy()
        hp[idx] += eps
        hm[idx] -= eps
        gh[idx] = (L(hp, W) - L(hm, W)) / (2 * eps)
    gW = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += eps
        Wm[idx] -= eps
        gW[idx] = (L(h, Wp) - L(h, Wm)) / (2 * eps)
    np.testing.assert_allclose(r["grad_h"], gh, rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(r["grad_W"], gW, rtol=1e-6, atol=1e-9)


# ------------------------------------------- independent library composite

@pytest.mark.parametrize("T,m,reduction", [(0.0, 1.0, "mean"), (2.0, 0.5, "mean"), (1.0, 1.3, "sum")])
def test_torch_fp64_cross_entropy_and_autograd(T, m, reduction):
    torch = pytest.importorskip("torch")
    h, W, labels = _rand(16, 8, 33, seed=11, scale=0.7, n_ign=3)
    r = flce_reference(h, W, labels, IGN, T, m, reduction)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    logits = torch.nn.functional.linear(th, tW) * m
    if T > 0:
        logits = T * torch.tanh(logits / T)
    loss = torch.nn.functional.cross_entropy(logits, torch.tensor(labels), ignore_index=IGN,
                                             reduction=reduction)
    loss.backward()
    assert r["loss"] == pytest.approx(loss.item(), rel=1e-13)
    np.testing.assert_allclose(r["grad_h"], th.grad.numpy(), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(r["grad_W"], tW.grad.numpy(), rtol=1e-11, atol=1e-15)
    pred = torch.argmax(logits, dim=1).numpy()
    valid = labels != IGN
    assert r["n_correct"] == int(np.sum(valid & (pred == labels)))


@pytest.mark.parametrize("T,m", [(0.0, 1.0), (1.5, 0.6)])
def test_torch_fp64_reduction_none_with_row_gradients(T, m):
    torch = pytest.importorskip("torch")
    h, W, labels = _rand(14, 6, 29, seed=21, scale=0.8, n_ign=3)
    w = np.random.default_rng(5).normal(size=14)          # any sign
    r = flce_reference(h, W, labels, IGN, T, m, "none", grad_rows=w)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    logits = torch.nn.functional.linear(th, tW) * m
    if T > 0:
        logits = T * torch.tanh(logits / T)
    rows = torch.nn.functional.cross_entropy(logits, torch.tensor(labels), ignore_index=IGN,
                                             reduction="none")
    rows.backward(torch.tensor(w))
    np.testing.assert_allclose(r["loss_rows"], rows.detach().numpy(), rtol=1e-13, atol=1e-15)
    assert r["loss"] == pytest.approx(rows.detach().sum().item(), rel=1e-13)
    np.testing.assert_allclose(r["grad_h"], th.grad.numpy(), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(r["grad_W"], tW.grad.numpy(), rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_torch_fp64_upstream_scalar_gradient(reduction):
    torch = pytest.importorskip("torch")
    h, W, labels = _rand(12, 5, 17, seed=22, scale=0.9, n_ign=2)
    g = -0.37
    r = flce_reference(h, W, labels, IGN, 2.0, 0.8, reduction, grad_scale=g)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tW = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    logits = 2.0 * torch.tanh(torch.nn.functional.linear(th, tW) * 0.8 / 2.0)
    loss = torch.nn.functional.cross_entropy(logits, torch.tensor(labels), ignore_index=IGN,
                                             reduction=reduction)
    loss.backward(torch.tensor(g, dtype=torch.float64))
    np.testing.assert_allclose(r["grad_h"], th.grad.numpy(), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(r["grad_W"], tW.grad.numpy(), rtol=1e-11, atol=1e-15)


def test_row_gradients_are_linear_and_reduce_to_sum():
    h, W, labels = _rand(10, 4, 13, seed=23, scale=0.6, n_ign=2)
    rng = np.random.default_rng(6)
    w1, w2 = rng.normal(size=10), rng.normal(size=10)
    r1 = flce_reference(h, W, labels, IGN, 1.0, 1.0, "none", grad_rows=w1)
    r2 = flce_reference(h, W, labels, IGN, 1.0, 1.0, "none", grad_rows=w2)
    r12 = flce_reference(h, W, labels, IGN, 1.0, 1.0, "none", grad_rows=w1 - 3.0 * w2)
    for k in ("grad_h", "grad_W"):
        np.testing.assert_allclose(r12[k], r1[k] - 3.0 * r2[k], rtol=1e-10, atol=1e-13)
    rs = flce_reference(h, W, labels, IGN, 1.0, 1.0, "sum")
    rn = flce_reference(h, W, labels, IGN, 1.0, 1.0, "none")
    assert rn["loss"] == pytest.approx(rs["loss"], rel=1e-14)
    for k in ("grad_h", "grad_W"):
        np.testing.assert_allclose(rn[k], rs[k], rtol=1e-14, atol=1e-16)
    with pytest.raises(ValueError):
        flce_reference(h, W, labels, IGN, 1.0, 1.0, "mean", grad_rows=w1)


# ------------------------------------------- cross-entropy on given logits

@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_cross_entropy_on_logits_is_flce_with_identity_weight(reduction):
    # with W = I (H = V), m = 1 and no cap the logits are h itself, so the
    # cross-entropy of given logits must equal the fused definition and its
    # logit gradient must equal grad_h = dlogits @ I
    rng = np.random.default_rng(31)
    V = 23
    z = 2.0 * rng.standard_normal((17, V))
    labels = rng.integers(0, V, 17)
    labels[[2, 9]] = IGN
    ce = oracle.cross_entropy_on_logits(z, labels, IGN, reduction)
    fl = flce_reference(z, np.eye(V), labels, IGN, 0.0, 1.0, reduction)
    assert ce["loss"] == pytest.approx(fl["loss"], rel=1e-14)
    np.testing.assert_allclose(ce["grad_z"], fl["grad_h"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(ce["lse"], fl["lse"], rtol=1e-15)
    assert ce["n_correct"] == fl["n_correct"]


def test_cross_entropy_on_logits_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(32)
    z = 3.0 * rng.standard_normal((19, 41))
    labels = rng.integers(0, 41, 19)
    labels[[0, 5, 6]] = IGN
    w = rng.normal(size=19)
    ce = oracle.cross_entropy_on_logits(z, labels, IGN, "none", grad_rows=w)
    tz = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    rows = torch.nn.functional.cross_entropy(tz, torch.tensor(labels), ignore_index=IGN, reduction="none")
    rows.backward(torch.tensor(w))
    np.testing.assert_allclose(ce["loss_rows"], rows.detach().numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ce["grad_z"], tz.grad.numpy(), rtol=1e-12, atol=1e-16)


# --------------------------------------------------------------------- argmax

def test_brute_force_argmax_with_ties():
    rng = np.random.default_rng(12)
    N, H, V = 9, 2, 7
    # integer-valued logits so that ties occur and are exact
    h = rng.integers(-2, 3, (N, H)).astype(float)
    W = rng.integers(-2, 3, (V, H)).astype(float)
    labels = rng.integers(0, V, N)
    r = flce_reference(h, W, labels, IGN, 0.0, 1.0, "mean")
    for i in range(N):
        row = [sum(h[i, k] * W[v, k] for k in range(H)) for v in range(V)]
        best = 0
        for v in range(1, V):
            if row[v] > row[best]:
                best = v
        assert r["pred"][i] == best
        srt = sorted(row)
        assert r["margin"][i] == pytest.approx(srt[-1] - srt[-2], abs=1e-12)
    assert r["n_correct"] == sum(int(r["pred"][i] == labels[i]) for i in range(N))


def test_planted_labels_count():
    h, W, labels = _rand(40, 6, 25, seed=13, n_ign=4)
    r = flce_reference(h, W, labels, IGN, 0.0, 1.0, "mean")
    valid = labels != IGN
    rng = np.random.default_rng(14)
    plant = valid & (rng.random(40) < 0.5)
    lab2 = labels.copy()
    lab2[plant] = r["pred"][plant]
    r2 = flce_reference(h, W, lab2, IGN, 0.0, 1.0, "mean")
    assert r2["n_correct"] >= int(plant.sum())
    assert r2["n_correct"] == int(np.sum(valid & (r2["pred"] == lab2)))


def test_bad_label_raises():
    h, W, labels = _rand(4, 3, 5, seed=15, n_ign=0)
    labels[2] = 5
    with pytest.raises(ValueError):
        flce_reference(h, W, labels, IGN)


# ----------------------------------------- blocked / sampled forms vs full

@pytest.mark.parametrize("T,m,reduction", [(0.0, 1.0, "mean"), (1.0, 0.5, "sum")])
def test_sampled_forms_match_full(T, m, reduction):
    h, W, labels = _rand(50, 7, 37, seed=16, n_ign=5)
    r = flce_reference(h, W, labels, IGN, T, m, reduction)
    st = row_stats(h, W, labels, IGN, T, m, block=16)
    for k in ("M", "lse", "z_label", "margin", "loss_rows"):
        np.testing.assert_allclose(st[k], r[k], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(st["pred"], r["pred"])
    rows = np.array([0, 3, 17, 49])
    gh = grad_h_rows(h, W, labels, rows, r["n_valid"], IGN, T, m, reduction)
    np.testing.assert_allclose(gh, r["grad_h"][rows], rtol=1e-12, atol=1e-16)
    vrows = np.array([0, 5, 36] + [int(labels[labels != IGN][0])])
    gw = grad_W_rows(h, W, labels, vrows, st["lse"], r["n_valid"], IGN, T, m, reduction, block=8)
    np.testing.assert_allclose(gw, r["grad_W"][vrows], rtol=1e-12, atol=1e-16)


def test_window():
    pred = np.array([1, 2, 3, 4])
    labels = np.array([1, 2, 0, 4])
    margin = np.array([1.0, 0.001, 0.5, 0.002])
    M = np.array([5.0, 5.0, 5.0, 5.0])
    z_label = np.array([5.0, 5.0, 1.0, 4.995])
    valid = np.array([True, True, True, True])
    lo, hi = oracle.n_correct_window(pred, margin, z_label, M, labels, valid)
    assert (lo, hi) == (1, 3)
