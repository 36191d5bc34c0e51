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
    # N_valid from the workspace, and token accuracy n_correct / N_valid, for both entry points
    n_valid = int(np.sum(case.labels != IGN))
    for res in (f, o):
        assert int(res.n_valid.item()) == n_valid
        assert float(L.token_accuracy(res).item()) == int(res.n_correct.item()) / max(n_valid, 1)
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
    assert int(fp.n_valid.item()) == int(op.n_valid.item()) == n_valid
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


@pytest.mark.parametrize("red", ["mean", "none"])
def test_batch_by_sequence_inputs_keep_their_shape(red):
    """[B, S, H] hidden states and [B, S] labels are flattened to rows and the
    outputs restored to the caller's shapes (SpecForge page, Changes): grad_h
    as [B, S, H], per-row losses as [B, S]; every value bitwise equal to the
    call on the flattened rows."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c4", 600, 256, 1000, 2.0, 0.5, "mean")
    log(f"[options] [B, S, H] inputs, reduction {red}")
    h, W, lab = to_device(case)
    h3, l3 = h.reshape(3, 200, 256), lab.reshape(3, 200)
    flat = L.fwd_bwd(h, W, lab, IGN, 2.0, 0.5, red)
    shaped = L.fwd_bwd(h3, W, l3, IGN, 2.0, 0.5, red)
    torch.cuda.synchronize()
    assert shaped.grad_h.shape == (3, 200, 256)
    assert torch.equal(shaped.grad_h.reshape(600, 256), flat.grad_h)
    assert torch.equal(shaped.grad_W, flat.grad_W)
    assert shaped.loss.item() == flat.loss.item() and shaped.n_correct.item() == flat.n_correct.item()
    f3 = L.forward(h3, W, l3, IGN, 2.0, 0.5, red)
    f1 = L.forward(h, W, lab, IGN, 2.0, 0.5, red)
    torch.cuda.synchronize()
    assert f3.loss.item() == f1.loss.item()
    if red == "none":
        assert shaped.loss_rows.shape == (3, 200) and f3.loss_rows.shape == (3, 200)
        assert torch.equal(shaped.loss_rows.reshape(-1), flat.loss_rows)
        assert torch.equal(f3.loss_rows.reshape(-1), f1.loss_rows)
    # the differentiable wrapper: gradients arrive in the inputs' shapes
    hh = h3.clone().requires_grad_(True)
    WW = W.clone().requires_grad_(True)
    loss, _ = L.linear_cross_entropy(hh, WW, l3, IGN, 2.0, 0.5, red)
    (loss.sum() if red == "none" else loss).backward()
    torch.cuda.synchronize()
    assert hh.grad.shape == (3, 200, 256) and WW.grad.shape == W.shape and WW.grad.dtype == W.dtype
    assert torch.equal(hh.grad.reshape(600, 256), flat.grad_h)
    ref = oracle.flce_reference(case.h_f32(), case.W_f32(), case.labels, IGN, 2.0, 0.5, red)
    _, gt = tolerances(case.cfg.dtype)
    assert rel_fro(WW.grad.float().cpu().numpy(), ref["grad_W"]) <= gt


def test_autograd_step_never_synchronises(monkeypatch):
    """The differentiable wrapper enqueues its forward, backward and gradient
    scaling without waiting for the device: the status reader (the library's
    one synchronising call) must not run.  The upstream gradient stays on the
    device and is applied in fp32 by flce_scale_grads; W's gradient comes back
    in W's dtype."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    from linear_cross_entropy_gemm_amd import torch_api

    def no_sync(*a, **k):
        raise AssertionError("flce_read_status called in the training step")

    case = make("c2", 600, 320, 1000, 1.0, 0.37, "mean")
    log("[options] autograd step without synchronisation")
    h, W, lab = to_device(case)
    monkeypatch.setattr(torch_api._lib, "flce_read_status", no_sync)
    hh = h.clone().requires_grad_(True)
    WW = W.clone().requires_grad_(True)
    g = torch.tensor(-1.7303, device=h.device)   # not representable in bf16
    loss, nc = L.linear_cross_entropy(hh, WW, lab, IGN, 1.0, 0.37)
    (loss * g).backward()
    monkeypatch.undo()
    torch.cuda.synchronize()
    ref = oracle.flce_reference(case.h_f32(), case.W_f32(), case.labels, IGN, 1.0, 0.37, "mean",
                                grad_scale=float(g.item()))
    lt, gt = tolerances(case.cfg.dtype)
    e_gh = rel_fro(hh.grad.float().cpu().numpy(), ref["grad_h"])
    e_gW = rel_fro(WW.grad.float().cpu().numpy(), ref["grad_W"])
    log(f"  grad_h {e_gh:.2e} grad_W {e_gW:.2e}")
    assert abs(loss.item() - ref["loss"]) / ref["loss"] <= lt
    assert e_gh <= gt and e_gW <= gt
    assert WW.grad.dtype == torch.bfloat16 and hh.grad.dtype == torch.bfloat16


def test_autograd_without_gradients_runs_forward_only():
    """With no input needing a gradient the wrapper runs flce_fwd: the same
    loss and n_correct bitwise, and no [V, H] accumulator."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c4", 513, 448, 2100, 30.0, 0.5, "mean")
    h, W, lab = to_device(case)
    full = L.fwd_bwd(h, W, lab, IGN, 30.0, 0.5)
    with torch.no_grad():
        loss, nc = L.linear_cross_entropy(h, W, lab, IGN, 30.0, 0.5)
    torch.cuda.synchronize()
    assert loss.item() == full.loss.item() and nc.item() == full.n_correct.item()
    assert not loss.requires_grad


def test_scale_grads_matches_torch():
    """flce_scale_grads against plain torch on the same stored gradients:
    fp32 products, one rounding to the output dtype (bitwise), in place and
    out of place, with ragged element counts."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(5)
    for n_h, n_W in [(1003, 4099), (8, 16), (0, 77), (129, 0)]:
        gh = torch.from_numpy(rng.normal(size=n_h).astype(np.float32)).to(dev).bfloat16()
        gW = torch.from_numpy(rng.normal(size=n_W).astype(np.float32)).to(dev)
        for gv in (-1.7303, 1.0, 0.0, 3.0e-3):
            g = torch.tensor(gv, device=dev)
            oh, oW = L.scale_grads(g, gh if n_h else None, gW if n_W else None, torch.bfloat16)
            torch.cuda.synchronize()
            if n_h:
                assert torch.equal(oh, (gh.float() * g).bfloat16())
            if n_W:
                assert torch.equal(oW, (gW * g).bfloat16())
                _, o32 = L.scale_grads(g, None, gW, torch.float32)
                assert torch.equal(o32, gW * g)
        # in place (the raw call): grad_h_out = grad_h_in
        x = gh.clone()
        g = torch.tensor([0.5], device=dev)
        rc = L.flce_scale_grads(g.data_ptr(), x.data_ptr() if n_h else None, x.data_ptr() if n_h else None, n_h,
                                L.FLCE_DTYPE_BF16, None, None, 0, L.FLCE_DTYPE_F32,
                                torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert rc == L.FLCE_OK
        assert torch.equal(x, (gh.float() * 0.5).bfloat16())


def test_zero_upstream_gradient_gives_zero_gradients():
    """grad_scale = 0 is an upstream gradient of zero: grad_h and this call's
    grad_W term are zero (accumulation leaves grad_W as it was)."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c2", 600, 320, 1000, 1.0, 0.37, "mean")
    h, W, lab = to_device(case)
    o = L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, grad_scale=0.0)
    torch.cuda.synchronize()
    assert o.grad_h.abs().max().item() == 0.0 and o.grad_W.abs().max().item() == 0.0
    before = torch.randn_like(o.grad_W)
    o.grad_W.copy_(before)
    L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, out=o, accumulate_grad_W=True, grad_scale=0.0)
    torch.cuda.synchronize()
    assert torch.equal(o.grad_W, before)


def test_reused_outputs_of_another_call_are_rejected():
    """An output set whose buffers do not match the call (a smaller N, V or H,
    grad_W in bf16, a strided view) is rejected before anything is enqueued,
    and the buffers stay as they were."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c2", 600, 320, 1000, 1.0, 0.37, "mean")
    h, W, lab = to_device(case)
    o = L.fwd_bwd(h[:300], W[:500], lab[:300].clamp(max=499), IGN, 1.0, 0.37)
    torch.cuda.synchronize()
    snap = (o.grad_h.clone(), o.grad_W.clone())
    with pytest.raises(ValueError):
        L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, out=o)                       # larger N and V
    o2 = L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37)
    bad = [dict(grad_W=o2.grad_W.bfloat16()), dict(grad_W=o2.grad_W.t()), dict(grad_h=o2.grad_h[:, :160]),
           dict(n_correct=o2.n_correct.float()), dict(loss=o2.loss.reshape(1))]
    for kw in bad:
        import dataclasses
        with pytest.raises(ValueError):
            L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, out=dataclasses.replace(o2, **kw))
    torch.cuda.synchronize()
    assert torch.equal(o.grad_h, snap[0]) and torch.equal(o.grad_W, snap[1])
    with pytest.raises(ValueError):
        L.fwd_bwd(h, W, lab, IGN, 1.0, 0.37, workspace=torch.empty(16, dtype=torch.uint8, device=h.device))
