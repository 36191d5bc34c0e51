"""GPU parity of the materialised-logits path (``flce_logits`` and
``flce_cross_entropy``) against the fp64 oracle, through the C ABI:

* logits z = cap(m h W^T): relative Frobenius error <= 5e-3 (bf16 storage:
  one rounding of 2^-9 relative per element) / 1e-5 (fp32), and the padding
  columns of a row-padded output are left untouched;
* cross-entropy of given logits: the oracle runs on exactly the values the
  GPU reads (the stored logits widened to fp64), so loss, per-row loss and
  log-sum-exp agree to 1e-5 for both dtypes; the logit gradient to 1e-2
  (bf16 storage of the gradient) / 1e-5 relative Frobenius; argmax exact on
  rows whose top-2 margin exceeds 1e-2; the in-place gradient equals the
  out-of-place one bitwise;
* the materialised path and the fused path give the same loss (bf16: within
  2e-3 relative, the logits being rounded to bf16 before the loss).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import log, rel_fro, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]

IGN = synth.IGNORE_INDEX

# (id, base, N, H, V, T, m, reduction)
SHAPES = [
    ("bf16_T1_ragged", "c2", 600, 320, 1000, 1.0, 0.37, "mean"),
    ("bf16_V_odd", "c4", 300, 256, 777, 30.0, 0.5, "sum"),
    ("f32_nocap", "c1", 257, 96, 530, 0.0, 1.0, "mean"),
    ("bf16_tiny_vocab", "c2", 90, 64, 37, 2.0, 1.0, "mean"),
]


def make(base, N, H, V, T, m, red):
    kw = dict(softcap_T=T, multiplier=m, reduction=red)
    if synth.CONFIGS[base].seq_len:
        kw["seq_len"] = max(1, N // 4)
    return synth.make_case(synth.small_config(base, **kw), N=N, H=H, V=V)


@pytest.mark.parametrize("cid,base,N,H,V,T,m,red", SHAPES, ids=[s[0] for s in SHAPES])
def test_logits_and_cross_entropy(cid, base, N, H, V, T, m, red):
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make(base, N, H, V, T, m, red)
    log(f"[logits] {cid}: N={N} H={H} V={V} T={T} m={m} {red}")
    h, W, lab = to_device(case)
    cap = T if T > 0 else None
    # logits into a row-padded buffer whose padding holds a sentinel
    per = 16 // h.element_size()
    ld = (V + per - 1) // per * per + per
    buf = torch.full((N, ld), 7.0, dtype=h.dtype, device=h.device)
    z = L.logits(h, W, cap, m, out=buf)
    torch.cuda.synchronize()
    _, zref = oracle.capped_logits(case.h_f32(), case.W_f32(), m, T)
    tol_z = 1e-5 if case.cfg.dtype == "f32" else 5e-3
    e_z = rel_fro(z.float().cpu().numpy(), zref)
    log(f"  logits rel {e_z:.2e}")
    assert e_z <= tol_z
    assert torch.all(buf[:, V:] == 7.0)

    # cross-entropy of exactly these logits
    zg = z.float().cpu().numpy().astype(np.float64)
    ce_ref = oracle.cross_entropy_on_logits(zg, case.labels, IGN, red)
    o = L.cross_entropy(z, lab, IGN, red, grad=True, row_outputs=True)
    torch.cuda.synchronize()
    e_loss = abs(o.loss.item() - ce_ref["loss"]) / abs(ce_ref["loss"])
    lr = o.loss_rows.cpu().numpy().astype(np.float64)
    ls = o.lse_rows.cpu().numpy().astype(np.float64)
    e_rows = float(np.max(np.abs(lr - ce_ref["loss_rows"]) / np.maximum(np.abs(ce_ref["loss_rows"]), 1.0)))
    e_lse = float(np.max(np.abs(ls - ce_ref["lse"]) / np.maximum(np.abs(ce_ref["lse"]), 1.0)))
    tol_g = 1e-5 if case.cfg.dtype == "f32" else 1e-2
    e_g = rel_fro(o.grad_logits.float().cpu().numpy(), ce_ref["grad_z"])
    sure = ce_ref["margin"] > 1e-2
    pr = o.pred_rows.cpu().numpy()
    log(f"  ce: loss rel {e_loss:.2e}, rows {e_rows:.2e}, lse {e_lse:.2e}, grad {e_g:.2e}, "
        f"n_correct {int(o.n_correct.item())} ref {ce_ref['n_correct']}")
    assert e_loss <= 1e-5 and e_rows <= 1e-5 and e_lse <= 1e-5
    assert e_g <= tol_g
    assert np.array_equal(pr[sure], ce_ref["pred"][sure])
    lo, hi = oracle.n_correct_window(ce_ref["pred"], ce_ref["margin"], ce_ref["z_label"], ce_ref["M"],
                                     case.labels, ce_ref["valid"])
    assert lo <= int(o.n_correct.item()) <= hi
    gz = o.grad_logits.float().cpu().numpy()
    assert np.all(gz[case.labels == IGN] == 0.0)

    # in place: the same gradient, written over the logits
    zc = buf.clone()
    zin = zc[:, :V]
    o2 = L.cross_entropy(zin, lab, IGN, red, grad=True, in_place=True)
    torch.cuda.synchronize()
    assert o2.loss.item() == o.loss.item()
    assert torch.equal(zin, o.grad_logits)
    vpad = (V + per - 1) // per * per              # the gradient's last 16-byte vector ends here
    assert torch.all(zc[:, V:vpad] == 0.0)
    assert torch.all(zc[:, vpad:] == 7.0)

    # materialised and fused paths agree on the loss
    f = L.forward(h, W, lab, IGN, cap, m, red)
    torch.cuda.synchronize()
    tol_f = 1e-5 if case.cfg.dtype == "f32" else 2e-3
    e_f = abs(f.loss.item() - o.loss.item()) / abs(f.loss.item())
    log(f"  fused vs materialised loss rel {e_f:.2e}")
    assert e_f <= tol_f


def test_cross_entropy_reduction_none_row_gradients():
    import torch
    import linear_cross_entropy_gemm_amd as L
    case = make("c2", 300, 128, 500, 0.0, 1.0, "mean")
    h, W, lab = to_device(case)
    z = L.logits(h, W)
    w = np.random.default_rng(9).normal(size=300).astype(np.float32)
    o = L.cross_entropy(z, lab, IGN, "none", grad=True, grad_rows=torch.from_numpy(w).to(h.device))
    torch.cuda.synchronize()
    ref = oracle.cross_entropy_on_logits(z.float().cpu().numpy().astype(np.float64), case.labels, IGN, "none",
                                         grad_rows=w.astype(np.float64))
    e_g = rel_fro(o.grad_logits.float().cpu().numpy(), ref["grad_z"])
    e_r = float(np.max(np.abs(o.loss_rows.cpu().numpy() - ref["loss_rows"]) / np.maximum(np.abs(ref["loss_rows"]), 1)))
    log(f"[logits] none: rows {e_r:.2e} grad {e_g:.2e}")
    assert e_r <= 1e-5 and e_g <= 1e-2


@pytest.mark.parametrize("m,T", [(0.5, 30.0), (-0.37, 1.0), (1.0, 2.0), (1.0, 1.5e-5), (0.5, 0.0)])
def test_softcap_on_the_gpu_matches_float64_tanh(m, T):
    """The kernels' softcap (Muse Glimmer page, Details > Softcap) on chosen raw
    logits: fp32 h rows [x, 0, 0, 0] against W rows [2^k, 0, 0, 0] make every
    raw logit exactly x 2^k, so flce_logits returns T tanh(m x 2^k / T) as the
    hardware computes it (exp2 and reciprocal instructions included).  Against
    float64 tanh on the same float32 inputs: relative error <= 1e-6 over
    |m a / T| from 1e-7 to 20, across the switch between the series and the
    exponential form, for both signs (host bound 4e-7, tests/test_softcap_host.py,
    plus the hardware approximations); exact zero at 0."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    dev = torch.device("cuda", 0)
    s = abs(np.float32(m) / np.float32(T)) if T > 0 else abs(np.float32(m))
    x = np.concatenate([np.linspace(0.0, 20.0, 3001), np.logspace(-7, 1.3, 1000), [0.25]])
    x = np.concatenate([x, -x])
    base_a = (x / s).astype(np.float32)
    ks = np.arange(-2, 6)                     # W rows 2^k: the raw logit is x * 2^k / s exactly
    h = np.zeros((base_a.size, 4), np.float32)
    h[:, 0] = base_a
    Wm = np.zeros((ks.size, 4), np.float32)
    Wm[:, 0] = np.exp2(ks).astype(np.float32)
    z = L.logits(torch.from_numpy(h).to(dev), torch.from_numpy(Wm).to(dev), T if T > 0 else None, m)
    torch.cuda.synchronize()
    z = z.cpu().numpy().astype(np.float64)
    a = base_a.astype(np.float64)[:, None] * np.exp2(ks)[None, :]
    m64, T64 = float(np.float32(m)), float(np.float32(T))
    ref = T64 * np.tanh(m64 * a / T64) if T > 0 else m64 * a
    nz = ref != 0.0
    rel = np.abs(z[nz] - ref[nz]) / np.abs(ref[nz])
    log(f"[softcap] m={m} T={T}: max rel {rel.max():.2e} over {nz.sum()} logits")
    assert np.all(np.isfinite(z))
    assert np.all(z[~nz] == 0.0)
    assert rel.max() <= (1e-6 if T > 0 else 0.0)
