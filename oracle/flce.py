"""Plain fp64 definition of fused linear cross-entropy (FLCE).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources.  What FLCE computes comes from two Liger-Kernel commit pages:

* commit e6a81bb0c3 ("Muse Glimmer"), Summary item 1: the fused linear +
  cross-entropy ("skip-logits") loss path, which never builds the
  [batch, seq, vocab] logits tensor; Summary item 2: token accuracy
  (argmax == label); Details > Softcap: the logits are capped as
  T * tanh(logits * m / T) with m the output multiplier, and because
  (m h) W^T = m (h W^T) the multiplier may equally scale the hidden states;
  Memory: the weight gradient is accumulated in fp32, [vocab, hidden].
* commit 40a9d8a61b ("DeepSeek-V3"), Summary: in training with labels the
  logits are never materialised and the loss runs through the fused path;
  Memory: chunked transients replace the logits, plus a fixed fp32
  weight-gradient accumulator.

Cross-entropy with ``ignore_index`` masking, mean over non-ignored rows or
sum, and its gradient softmax - onehot, are the standard definitions those
pages rely on.  Readings where the pages are silent:

* mean reduction divides by the number of non-ignored rows of the call; with
  no such row the loss is 0 and every gradient is 0;
* ``softcap_T <= 0`` means no softcap; m multiplies the raw logits before the
  cap, and with no cap the logits are m * (h W^T);
* the argmax is taken over the capped logits and the lowest index wins ties;
* ``grad_h`` is the gradient with respect to the caller's (un-multiplied) h
  and ``grad_W`` the gradient of this call alone (not accumulated across
  calls); the upstream gradient of the scalar loss is ``grad_scale``
  (default 1);
* reduction "none" keeps the per-row losses (``loss_rows``; the scalar
  ``loss`` is then their sum) and takes the upstream gradient of row i's loss
  from ``grad_rows[i]`` (default 1 for every row), as torch's
  ``cross_entropy(..., reduction="none")`` backward does.  The per-row
  outputs answer the predicted-tokens contract of the Muse Glimmer page
  (Testing Done) and the DeepSeek-V3 page (Summary).

Every array is float64.  bf16 and fp32 inputs widen to float64 exactly.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def reduction_scale(n_valid: int, reduction: str) -> float:
    """s: 1/N_valid for "mean" (0 when nothing is valid), 1 for "sum" and
    "none"."""
    if reduction == "mean":
        return 1.0 / n_valid if n_valid > 0 else 0.0
    if reduction in ("sum", "none"):
        return 1.0
    raise ValueError(f"unknown reduction {reduction!r}")


def row_weights(N: int, n_valid: int, reduction: str, grad_rows=None, grad_scale: float = 1.0):
    """Upstream gradient of each row's loss: s * grad_scale, times
    grad_rows[i] with reduction "none"."""
    w = np.full(N, reduction_scale(n_valid, reduction) * float(grad_scale))
    if grad_rows is not None:
        if reduction != "none":
            raise ValueError("grad_rows needs reduction 'none'")
        w = w * _f64(grad_rows).reshape(N)
    return w


def _valid_mask(labels: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    labels = np.asarray(labels)
    valid = labels != ignore_index
    bad = valid & ((labels < 0) | (labels >= V))
    if np.any(bad):
        raise ValueError("label outside [0, V) that is not ignore_index")
    return valid


def capped_logits(h, W, multiplier: float = 1.0, softcap_T: float = 0.0):
    """Return (a, z) for rows of h: a = m * (h W^T), z = T tanh(a / T) or a.

    Muse Glimmer page, Details > Softcap: logits are capped as
    T * tanh(logits * m / T).
    """
    a = float(multiplier) * (_f64(h) @ _f64(W).T)
    if softcap_T > 0:
        z = softcap_T * np.tanh(a / softcap_T)
    else:
        z = a
    return a, z


def _row_quantities(z: np.ndarray):
    """Row max, log-sum-exp (exact two-pass), argmax (lowest index) and the
    gap between the largest and second-largest logit."""
    M = z.max(axis=1)
    lse = M + np.log(np.exp(z - M[:, None]).sum(axis=1))
    pred = np.argmax(z, axis=1)          # first maximal index
    if z.shape[1] >= 2:
        second = np.partition(z, -2, axis=1)[:, -2]
        margin = M - second
    else:
        margin = np.full(z.shape[0], np.inf)
    return M, lse, pred, margin


def _dlogits(z, a, lse, labels, valid, s, softcap_T):
    """d loss / d a for a block of rows.

    d loss / d z = s * (softmax(z) - onehot(label)) on valid rows, 0 on ignored
    rows; chained through the softcap, dz/da = 1 - tanh^2(a / T).  ``s`` is a
    scalar or one weight per row.
    """
    p = np.exp(z - lse[:, None])
    dz = p
    rows = np.nonzero(valid)[0]
    dz[rows, labels[rows]] -= 1.0
    dz *= np.asarray(s)[:, None] if np.ndim(s) == 1 else s
    dz[~valid] = 0.0
    if softcap_T > 0:
        dz *= 1.0 - np.tanh(a / softcap_T) ** 2
    return dz


def flce_reference(h, W, labels, ignore_index: int = -100, softcap_T: float = 0.0,
                   multiplier: float = 1.0, reduction: str = "mean", grad_rows=None,
                   grad_scale: float = 1.0) -> dict:
    """Full forward and backward of FLCE for shapes that fit as one [N, V]
    array.  Returns loss, grad_h, grad_W, n_correct and per-row quantities."""
    h = _f64(h)
    W = _f64(W)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = h.shape[0], W.shape[0]
    valid = _valid_mask(labels, V, ignore_index)
    n_valid = int(valid.sum())
    s = reduction_scale(n_valid, reduction)
    w = row_weights(N, n_valid, reduction, grad_rows, grad_scale)
    a, z = capped_logits(h, W, multiplier, softcap_T)
    M, lse, pred, margin = _row_quantities(z)
    safe = np.where(valid, labels, 0)
    z_label = z[np.arange(N), safe]
    loss_rows = np.where(valid, lse - z_label, 0.0)
    loss = s * loss_rows.sum()
    correct = valid & (pred == labels)
    da = _dlogits(z, a, lse, safe, valid, w, softcap_T)
    grad_h = float(multiplier) * (da @ W)
    grad_W = float(multiplier) * (da.T @ h)
    return dict(loss=loss, grad_h=grad_h, grad_W=grad_W, n_correct=int(correct.sum()),
                n_valid=n_valid, scale=s, lse=lse, M=M, z_label=z_label, pred=pred,
                margin=margin, loss_rows=loss_rows, valid=valid, z=z, dlogits=da)


def row_stats(h, W, labels, ignore_index: int = -100, softcap_T: float = 0.0,
              multiplier: float = 1.0, rows=None, block: int = 256) -> dict:
    """Per-row M, lse, z_label, pred and margin for ``rows`` (default all),
    over the full vocabulary, computed in independent blocks of rows.

    W may be passed already widened to float64 to avoid repeated conversion.
    """
    W64 = _f64(W)
    labels = np.asarray(labels, dtype=np.int64)
    V = W64.shape[0]
    rows = np.arange(h.shape[0]) if rows is None else np.asarray(rows)
    valid = _valid_mask(labels[rows], V, ignore_index)
    out = {k: np.empty(len(rows)) for k in ("M", "lse", "z_label", "margin")}
    out["pred"] = np.empty(len(rows), dtype=np.int64)
    for b0 in range(0, len(rows), block):
        r = rows[b0:b0 + block]
        _, z = capped_logits(h[r], W64, multiplier, softcap_T)
        M, lse, pred, margin = _row_quantities(z)
        lab = np.where(valid[b0:b0 + block], labels[r], 0)
        out["M"][b0:b0 + len(r)] = M
        out["lse"][b0:b0 + len(r)] = lse
        out["pred"][b0:b0 + len(r)] = pred
        out["margin"][b0:b0 + len(r)] = margin
        out["z_label"][b0:b0 + len(r)] = z[np.arange(len(r)), lab]
    out["valid"] = valid
    out["loss_rows"] = np.where(valid, out["lse"] - out["z_label"], 0.0)
    return out


def grad_h_rows(h, W, labels, rows, n_valid: int, ignore_index: int = -100,
                softcap_T: float = 0.0, multiplier: float = 1.0,
                reduction: str = "mean") -> np.ndarray:
    """grad_h for the selected rows: m * sum_v dlogits[i, v] * W[v, :].

    Row-local: each row needs only its own logits (and the global N_valid for
    the mean scale)."""
    W64 = _f64(W)
    labels = np.asarray(labels, dtype=np.int64)
    rows = np.asarray(rows)
    V = W64.shape[0]
    valid = _valid_mask(labels[rows], V, ignore_index)
    s = reduction_scale(n_valid, reduction)
    a, z = capped_logits(h[rows], W64, multiplier, softcap_T)
    _, lse, _, _ = _row_quantities(z)
    da = _dlogits(z, a, lse, np.where(valid, labels[rows], 0), valid, s, softcap_T)
    return float(multiplier) * (da @ W64)


def grad_W_rows(h, W, labels, vocab_rows, lse, n_valid: int, ignore_index: int = -100,
                softcap_T: float = 0.0, multiplier: float = 1.0,
                reduction: str = "mean", block: int = 4096) -> np.ndarray:
    """grad_W for the selected vocabulary rows: m * sum_i dlogits[i, v] h[i, :].

    Needs the log-sum-exp of every row (``lse``, from ``row_stats``), because
    each vocabulary row's gradient sums over all tokens."""
    h64 = _f64(h)
    labels = np.asarray(labels, dtype=np.int64)
    vocab_rows = np.asarray(vocab_rows)
    V = np.asarray(W).shape[0]
    valid = _valid_mask(labels, V, ignore_index)
    s = reduction_scale(n_valid, reduction)
    Wv = _f64(np.asarray(W)[vocab_rows])
    out = np.zeros((len(vocab_rows), h64.shape[1]))
    lse = _f64(lse)
    for b0 in range(0, h64.shape[0], block):
        sl = slice(b0, b0 + block)
        a = float(multiplier) * (h64[sl] @ Wv.T)             # [rows, S]
        z = softcap_T * np.tanh(a / softcap_T) if softcap_T > 0 else a
        p = np.exp(z - lse[sl, None])
        onehot = (labels[sl, None] == vocab_rows[None, :]) & valid[sl, None]
        dz = s * (p - onehot)
        dz[~valid[sl]] = 0.0
        if softcap_T > 0:
            dz *= 1.0 - np.tanh(a / softcap_T) ** 2
        out += dz.T @ h64[sl]
    return float(multiplier) * out


def cross_entropy_on_logits(z, labels, ignore_index: int = -100, reduction: str = "mean",
                            grad_rows=None, grad_scale: float = 1.0) -> dict:
    """Cross-entropy of already materialised (and already capped) logits
    z [N, V]: the non-fused branch the Liger-Kernel pages compare against
    (Muse Glimmer page, Testing Done: the non-fused softcap branch;
    DeepSeek-V3 page, Summary: with logits materialised the plain loss
    function is used).  Returns the loss, per-row quantities and the gradient
    with respect to z (softmax - onehot, scaled like the fused path; no
    softcap derivative, since z is the input here)."""
    z = _f64(z)
    labels = np.asarray(labels, dtype=np.int64)
    N, V = z.shape
    valid = _valid_mask(labels, V, ignore_index)
    n_valid = int(valid.sum())
    s = reduction_scale(n_valid, reduction)
    w = row_weights(N, n_valid, reduction, grad_rows, grad_scale)
    M, lse, pred, margin = _row_quantities(z)
    safe = np.where(valid, labels, 0)
    z_label = z[np.arange(N), safe]
    loss_rows = np.where(valid, lse - z_label, 0.0)
    grad_z = _dlogits(z.copy(), z, lse, safe, valid, w, 0.0)
    return dict(loss=s * loss_rows.sum(), loss_rows=loss_rows, lse=lse, pred=pred, M=M, margin=margin,
                z_label=z_label, valid=valid, n_valid=n_valid,
                n_correct=int(np.sum(valid & (pred == labels))), grad_z=grad_z)


def n_correct_window(pred, margin, z_label, M, labels, valid, tol: float = 1e-2):
    """Range [lo, hi] that a correct n_correct must fall in.

    Rows whose top-2 gap exceeds ``tol`` have one argmax and count exactly;
    rows within ``tol`` of a tie may count either way if their label is among
    the near-maximal logits."""
    pred = np.asarray(pred)
    labels = np.asarray(labels)
    valid = np.asarray(valid, dtype=bool)
    clear = valid & (np.asarray(margin) > tol)
    lo = int(np.sum(clear & (pred == labels)))
    near = valid & ~clear & (np.asarray(z_label) >= np.asarray(M) - tol)
    return lo, lo + int(np.sum(near))
