"""GPU parity of the forward-only entry point and of the call options against
the fp64 oracle (through the C ABI):

* ``flce_fwd``: loss, n_correct and the per-row loss / log-sum-exp / argmax
  against the oracle, and bitwise against ``flce_fwd_bwd_ex`` on the same
  inputs (the same kernels compute every row's statistics);
* reduction "none" with per-row upstream gradients of any sign;
* a scalar upstream gradient (``grad_scale``);
* accumulation into a pre-filled grad_W, including N = 0;
* the autograd wrapper with reduction "none".

Tolerances as in test_parity_gpu: loss (and each row loss, relative to
max(|ref|, 1)) 1e-5 fp32 / 2e-3 bf16; gradients 1e-4 / 2e-2 relative
Frobenius; argmax exact on rows whose top-2 margin exceeds 1e-2.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, rel_fro, to_device, tolerances

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]

IGN = synth.IGNORE_INDEX

# (id, base, N, H, V, T, m, reduction)
SHAPES = [
    ("bf16_T1", "c2", 600, 320, 1000, 1.0, 0.37, "mean"),
    ("bf16_T30_sum", "c4", 513, 448, 2100, 30.0, 0.5, "sum"),
    ("f32_nocap", "c1", 300, 96, 530, 0.0, 1.0, "mean"),
    ("bf16_tiny_vocab", "c2", 90, 64, 37, 2.0, 1.0, "mean"),
]


def make(base, N, H, V, T, m, red, seed=None):
    kw = dict(softcap_T=T, multiplier=m, reduction=red)
    if synth.CONFIGS[base].seq_len:
        kw["seq_len"] = max(1, N // 4)
    return synth.make_case(synth.small_config(base, **kw), N=N, H=H, V=V, seed=seed)


def softcap(case):
    return case.cfg.softcap_T if case.cfg.softcap_T > 0 else None


def check_rows(case, ref, loss_rows, lse_rows, pred_rows):
    lt, _ = tolerances(case.cfg.dtype)
    lr = loss_rows.cpu().numpy().astype(np.float64)
    ls = lse_rows.cpu().numpy().astype(np.float64)
    pr = pred_rows.cpu().numpy()
    e_lr = np.max(np.abs(lr - ref["loss_rows"]) / np.maximum(np.abs(ref["loss_rows"]), 1.0))
    e_ls = np.max(np.abs(ls - ref["lse"]) / np.maximum(np.abs(ref["lse"]), 1.0))
    sure = ref["margin"] > 1e-2
    log(f"  rows: loss rel {e_lr:.2e}, lse rel {e_ls:.2e}, argmax exact on {int(sure.sum())} of {len(pr)} rows")
    assert e_lr <= lt and e_ls <= lt
    assert np.all(lr[case.labels == IGN] == 0.0)
    assert np.array_equal(pr[sure], ref["pred"][sure])
    assert np.all((pr >= 0) & (pr < case.W.shape[0]))


@pytest.mark.parametrize("cid,base,N,H,V,T,m,red", SHAPES, ids=[s[0] for s in SHAPES])
def test_forward_only(cid, base, N, H, V, T, m, red):
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make(base, N, H, V, T, m, red)
    log(f"[options] forward only {cid}: N={N} H={H} V={V} T={T} m={m} {red}")
    h, W, lab = to_device(case)
    f = L.forward(h, W, lab, IGN, softcap(case), m, red, row_outputs=True)
    o = L.fwd_bwd(h, W, lab, IGN, softcap(case), m, red, row_outputs=True)
    torch.cuda.synchronize()
    ref = oracle.flce_reference(case.h_f32(), case.W_f32(), case.labels, IGN, T, m, red)
    lt, _ = tolerances(case.cfg.dtype)
    loss = float(f.loss.item())
    log(f"  loss {loss:.8g} ref {ref['loss']:.8g}")
    assert abs(loss - ref["loss"]) / abs(ref["loss"]) <= lt
    lo, hi = oracle.n_correct_window(ref["pred"], ref["margin"], ref["z_label"], ref["M"], case.labels,
                                     ref["valid"])
    assert lo <= int(f.n_correct.item()) <= hi
    check_rows(case, ref, f.loss_rows, f.lse_rows, f.pred_rows)
    # the same kernels compute each row's statistics on both entry points
    assert f.loss.item() == o.loss.item()
    assert int(f.n_correct.item()) == int(o.n_correct.item())
    assert torch.equal(f.loss_rows, o.loss_rows)
    assert torch.equal(f.lse_rows, o.lse_rows)
    assert torch.equal(f.pred_rows, o.pred_rows)
    # without every row's lse / argmax the ignored rows are packed out: the
    # same per-row statistics, summed over the packed rows
    fp = L.forward(h, W, lab, IGN, softcap(case), m, red)
    op = L.fwd_bwd(h, W, lab, IGN, softcap(case), m, red)
    torch.cuda.synchronize()
    assert fp.lse_rows is None and fp.pred_rows is None
    assert fp.loss.item() == op.loss.item()
    assert int(fp.n_correct.item()) == int(f.n_correct.item()) == int(op.n_correct.item())
    assert abs(fp.loss.item() - loss) <= 1e-6 * abs(loss)


@pytest.mark.parametrize("cid,base,N,H,V,T,m,red", SHAPES[:3], ids=[s[0] for s in SHAPES[:3]])
def test_reduction_none_row_gradients(cid, base, N, H, V, T, m, red):
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make(base, N, H, V, T, m, red)
    log(f"[options] reduction none {cid}")
    h, W, lab = to_device(case)
    w = np.random.default_rng(77).normal(size=N).astype(np.float32)
    w[::7] = 0.0
    ref = oracle.flce_reference(case.h_f32(), case.W_f32(), case.labels, IGN, T, m, "none",
                                grad_rows=w.astype(np.float64))
    lt, gt = tolerances(case.cfg.dtype)
    # packed rows (row losses only) and all rows (with every row's lse / argmax)
    for row_outputs in (False, True):
        o = L.fwd_bwd(h, W, lab, IGN, softcap(case), m, "none", grad_rows=torch.from_numpy(w).to(h.device),
                      row_outputs=row_outputs)
        torch.cuda.synchronize()
        e_loss = abs(o.loss.item() - ref["loss"]) / abs(ref["loss"])
        e_gh = rel_fro(o.grad_h.float().cpu().numpy(), ref["grad_h"])
        e_gW = rel_fro(o.grad_W.cpu().numpy(), ref["grad_W"])
        log(f"  row_outputs={row_outputs}: sum of rows rel {e_loss:.2e} | grad_h {e_gh:.2e} grad_W {e_gW:.2e}")
        assert e_loss <= lt and e_gh <= gt and e_gW <= gt
        if row_outputs:
            check_rows(case, ref, o.loss_rows, o.lse_rows, o.pred_rows)
        else:
            assert o.lse_rows is None and o.pred_rows is None
            lr = o.loss_rows.cpu().numpy().astype(np.float64)
            assert np.max(np.abs(lr - ref["loss_rows"]) / np.maximum(np.abs(ref["loss_rows"]), 1.0)) <= lt
            assert np.all(lr[case.labels == IGN] == 0.0)
        gh = o.grad_h.float().cpu().numpy()
        assert np.all(gh[(case.labels == IGN) | (w == 0.0)] == 0.0)


def test_grad_scale_and_accumulate():
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c2", 600, 320, 1000, 1.0, 0.37, "mean")
    log("[options] grad_scale and accumulate_grad_W")
    h, W, lab = to_device(case)
    g = -2.5
    base = L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, "mean")
    scaled = L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, "mean", grad_scale=g)
    torch.cuda.synchronize()
    ref = oracle.flce_reference(case.h_f32(), case.W_f32(), case.labels, IGN, 1.0, 0.37, "mean",
                                grad_scale=g)
    _, gt = tolerances(case.cfg.dtype)
    e_gh = rel_fro(scaled.grad_h.float().cpu().numpy(), ref["grad_h"])
    e_gW = rel_fro(scaled.grad_W.cpu().numpy(), ref["grad_W"])
    log(f"  grad_scale {g}: grad_h {e_gh:.2e} grad_W {e_gW:.2e}")
    assert e_gh <= gt and e_gW <= gt
    assert scaled.loss.item() == base.loss.item()
    # grad_W += this call's term, on top of arbitrary stored values
    R = torch.from_numpy(np.random.default_rng(3).normal(size=tuple(base.grad_W.shape)).astype(np.float32))
    acc = L.FlceOutputs(loss=torch.empty((), device=h.device), grad_h=torch.empty_like(base.grad_h),
                        grad_W=R.to(h.device).clone(), n_correct=torch.empty((), dtype=torch.int64, device=h.device),
                        workspace=base.workspace)
    L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, "mean", out=acc, accumulate_grad_W=True, grad_scale=g)
    torch.cuda.synchronize()
    e_acc = rel_fro(acc.grad_W.cpu().numpy().astype(np.float64) - R.double().numpy(), ref["grad_W"])
    log(f"  accumulate: added term rel {e_acc:.2e}")
    assert e_acc <= gt
    # N = 0 with accumulation leaves grad_W untouched
    before = acc.grad_W.clone()
    empty = L.FlceOutputs(loss=torch.full((), 7.0, device=h.device), grad_h=h[:0].clone(),
                          grad_W=acc.grad_W, n_correct=torch.empty((), dtype=torch.int64, device=h.device),
                          workspace=base.workspace)
    L.fwd_bwd(h[:0], W, lab[:0], IGN, 1.0, 0.37, "mean", out=empty, accumulate_grad_W=True)
    torch.cuda.synchronize()
    assert torch.equal(acc.grad_W, before)
    assert empty.loss.item() == 0.0


def test_autograd_reduction_none():
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c4", 520, 256, 777, 2.0, 0.5, "mean")
    log("[options] autograd reduction none")
    h, W, lab = to_device(case)
    hh = h.clone().requires_grad_(True)
    WW = W.clone().requires_grad_(True)
    rows, nc = L.linear_cross_entropy(hh, WW, lab, IGN, 2.0, 0.5, "none")
    w = np.random.default_rng(8).normal(size=rows.shape[0]).astype(np.float32)
    (rows * torch.from_numpy(w).to(h.device)).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.flce_reference(case.h_f32(), case.W_f32(), case.labels, IGN, 2.0, 0.5, "none",
                                grad_rows=w.astype(np.float64))
    _, gt = tolerances(case.cfg.dtype)
    e_gh = rel_fro(hh.grad.float().cpu().numpy(), ref["grad_h"])
    e_gW = rel_fro(WW.grad.float().cpu().numpy(), ref["grad_W"])
    log(f"  grad_h {e_gh:.2e} grad_W {e_gW:.2e}")
    assert e_gh <= gt and e_gW <= gt
    assert rows.shape == lab.shape


def test_reused_outputs_gain_row_statistics():
    """An output set first filled without per-row statistics (reduction none:
    row losses only, valid rows packed) gets its log-sum-exp / argmax
    buffers when a later call on it asks for them."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c2", 600, 320, 1000, 1.0, 0.37, "mean")
    log("[options] reused outputs, then row statistics")
    h, W, lab = to_device(case)
    o = L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, "none")
    assert o.loss_rows is not None and o.lse_rows is None and o.pred_rows is None
    o = L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, "mean", out=o, row_outputs=True)
    torch.cuda.synchronize()
    ref = oracle.flce_reference(case.h_f32(), case.W_f32(), case.labels, IGN, 1.0, 0.37, "mean")
    check_rows(case, ref, o.loss_rows, o.lse_rows, o.pred_rows)
