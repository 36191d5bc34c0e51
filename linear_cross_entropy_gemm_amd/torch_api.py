"""PyTorch-facing wrappers: device memory and the current stream come from
torch; every step of the computation runs in ``flce_fwd_bwd_ex`` /
``flce_fwd``."""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.FLCE_DTYPE_BF16, torch.float32: _lib.FLCE_DTYPE_F32}
_REDUCTIONS = {"mean": _lib.FLCE_REDUCTION_MEAN, "sum": _lib.FLCE_REDUCTION_SUM,
               "none": _lib.FLCE_REDUCTION_NONE}


@dataclasses.dataclass
class FlceOutputs:
    loss: torch.Tensor        # [] fp32 (the sum of the row losses with reduction "none")
    grad_h: torch.Tensor      # [N, H] dtype of h
    grad_W: torch.Tensor      # [V, H] fp32
    n_correct: torch.Tensor   # [] int64
    workspace: torch.Tensor   # uint8, holds the status word
    loss_rows: Optional[torch.Tensor] = None   # [N] fp32 (row outputs / reduction "none")
    lse_rows: Optional[torch.Tensor] = None    # [N] fp32
    pred_rows: Optional[torch.Tensor] = None   # [N] int64, predicted token of every row
    n_valid: Optional[torch.Tensor] = None     # [] int64 view of the workspace: rows not ignored


@dataclasses.dataclass
class FlceForward:
    loss: torch.Tensor
    n_correct: torch.Tensor
    workspace: torch.Tensor
    loss_rows: Optional[torch.Tensor] = None
    lse_rows: Optional[torch.Tensor] = None
    pred_rows: Optional[torch.Tensor] = None
    n_valid: Optional[torch.Tensor] = None


def _n_valid_view(workspace: torch.Tensor) -> torch.Tensor:
    """N_valid of the last call that used ``workspace``, as a 0-d int64 view of
    the device memory the call wrote it to (FLCE_WS_N_VALID_OFFSET): no copy,
    no synchronisation; the next call on the workspace overwrites it."""
    o = _lib.WS_N_VALID_OFFSET
    return workspace[o:o + 8].view(torch.int64).reshape(())


def token_accuracy(out) -> torch.Tensor:
    """n_correct / N_valid (Muse Glimmer page, Summary item 2) of a ``fwd_bwd``
    or ``forward`` result, as a 0-d float64 device tensor (0 when every row is
    ignored); read it before the workspace is used again."""
    return out.n_correct.to(torch.float64) / torch.clamp(out.n_valid, min=1).to(torch.float64)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _prepare(h, W, labels, reduction):
    if h.dtype not in _DTYPES or W.dtype != h.dtype:
        raise TypeError(f"h and W must both be bfloat16 or float32 (got {h.dtype}, {W.dtype})")
    if not h.is_cuda or not W.is_cuda or not labels.is_cuda:
        raise ValueError("h, W and labels must be on the GPU")
    if reduction not in _REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    H = h.shape[-1]
    h2 = h.reshape(-1, H).contiguous()
    lab = labels.reshape(-1).to(torch.int64).contiguous()
    if lab.numel() != h2.shape[0]:
        raise ValueError("labels must have one entry per row of h")
    return h2, W.contiguous(), lab


def _workspace(workspace: Optional[torch.Tensor], nbytes: int, dev) -> torch.Tensor:
    """The caller's workspace (a contiguous uint8 tensor of at least ``nbytes``
    on the device of h), or a new one."""
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the device of h")
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, this call needs {nbytes}")
    return workspace


def _row_buffers(N: int, dev, want_loss: bool, want_stats: bool):
    """Per-row loss (reduction "none" or row_outputs) and per-row log-sum-exp /
    argmax (row_outputs only: asking for them keeps the ignored rows in the
    GEMMs, since those two are defined for every row)."""
    loss_rows = torch.empty(N, dtype=torch.float32, device=dev) if want_loss or want_stats else None
    if not want_stats:
        return loss_rows, None, None
    return loss_rows, torch.empty(N, dtype=torch.float32, device=dev), torch.empty(N, dtype=torch.int64, device=dev)


def _check_out(out: "FlceOutputs", N: int, H: int, V: int, h_dtype, dev) -> None:
    """Every buffer of a reused output set must match this call before its
    address reaches the kernels: shape, dtype, device and contiguity."""
    want = [("loss", out.loss, (), torch.float32), ("grad_h", out.grad_h, None, h_dtype),
            ("grad_W", out.grad_W, (V, H), torch.float32), ("n_correct", out.n_correct, (), torch.int64),
            ("loss_rows", out.loss_rows, (N,), torch.float32), ("lse_rows", out.lse_rows, (N,), torch.float32),
            ("pred_rows", out.pred_rows, (N,), torch.int64)]
    for name, t, shape, dt in want:
        if t is None:
            if name in ("loss", "grad_h", "grad_W", "n_correct"):
                raise ValueError(f"out.{name} is missing")
            continue
        if name == "grad_h":   # any shape of N x H elements with rows of H (restored to h's shape)
            ok_shape = t.dim() >= 1 and t.numel() == N * H and t.shape[-1] == H
        else:
            ok_shape = tuple(t.shape) == shape
        if not ok_shape:
            raise ValueError(f"out.{name} has shape {tuple(t.shape)}, this call needs "
                             f"{(N, H) if shape is None else shape}")
        if t.dtype != dt:
            raise ValueError(f"out.{name} is {t.dtype}, this call needs {dt}")
        if t.device != dev:
            raise ValueError(f"out.{name} is on {t.device}, this call runs on {dev}")
        if not t.is_contiguous():
            raise ValueError(f"out.{name} must be contiguous")


def fwd_bwd(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100,
            softcap: Optional[float] = None, multiplier: float = 1.0, reduction: str = "mean",
            workspace: Optional[torch.Tensor] = None, out: Optional[FlceOutputs] = None,
            check: bool = True, *, grad_rows: Optional[torch.Tensor] = None,
            grad_scale: Optional[float] = None, accumulate_grad_W: bool = False,
            row_outputs: bool = False) -> FlceOutputs:
    """One call of ``flce_fwd_bwd_ex`` on torch's current stream.

    ``h`` [..., H] is flattened to [N, H] and ``grad_h`` restored to its shape
    (SpecForge PR 1007, Changes: flatten rows for the vocabulary projection,
    then restore the output shape); with reduction "none" the per-row losses
    take the shape of ``labels``.  ``grad_rows`` (reduction "none") and
    ``grad_scale`` (None: 1; 0 gives zero gradients) are upstream gradients;
    with ``accumulate_grad_W`` the call adds its weight gradient to
    ``out.grad_W``.  A reused ``out`` must match the call (checked before the
    launch).  ``check`` synchronises the stream and raises on out-of-range
    labels; without it nothing waits and ``read_status(workspace)`` reports
    them later."""
    h2, Wc, lab = _prepare(h, W, labels, reduction)
    shape = h.shape
    N, H = h2.shape
    V = Wc.shape[0]
    dtype = _DTYPES[h.dtype]
    red = _REDUCTIONS[reduction]
    ws_bytes = _lib.flce_workspace_size(N, H, V, dtype, 0)
    if ws_bytes == 0:
        raise _lib.FlceError(_lib.FLCE_EUNSUPPORTED, "flce_workspace_size")
    dev = h.device
    if workspace is None and out is not None and out.workspace is not None \
            and out.workspace.device == dev and out.workspace.numel() >= ws_bytes:
        workspace = out.workspace   # a reused output set brings its workspace along
    workspace = _workspace(workspace, ws_bytes, dev)
    if accumulate_grad_W and out is None:
        raise ValueError("accumulate_grad_W needs out.grad_W holding the running sum")
    if out is None:
        out = FlceOutputs(
            loss=torch.empty((), dtype=torch.float32, device=dev),
            grad_h=torch.empty((N, H), dtype=h.dtype, device=dev),
            grad_W=torch.empty((V, H), dtype=torch.float32, device=dev),
            n_correct=torch.empty((), dtype=torch.int64, device=dev),
            workspace=workspace,
        )
    else:
        if out.loss_rows is not None:
            out.loss_rows = out.loss_rows.reshape(-1)
        _check_out(out, N, H, V, h.dtype, dev)
    want_rows = row_outputs or reduction == "none"
    if want_rows and out.loss_rows is None:
        out.loss_rows = torch.empty(N, dtype=torch.float32, device=dev)
    if row_outputs and out.lse_rows is None:
        out.lse_rows = torch.empty(N, dtype=torch.float32, device=dev)
    if row_outputs and out.pred_rows is None:
        out.pred_rows = torch.empty(N, dtype=torch.int64, device=dev)
    gr = None
    if grad_rows is not None:
        gr = grad_rows.reshape(-1).to(device=dev, dtype=torch.float32).contiguous()
        if gr.numel() != N:
            raise ValueError("grad_rows must have one entry per row")
    opts = _lib.flce_options_t(
        loss_rows=_ptr(out.loss_rows) if want_rows else None,
        lse_rows=_ptr(out.lse_rows) if row_outputs else None,
        pred_rows=_ptr(out.pred_rows) if row_outputs else None,
        grad_rows=_ptr(gr), grad_scale=float(grad_scale) if grad_scale is not None else 0.0,
        accumulate_grad_W=1 if accumulate_grad_W else 0, use_grad_scale=0 if grad_scale is None else 1)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _lib.flce_fwd_bwd_ex(_ptr(h2), _ptr(Wc), _ptr(lab), N, H, V, int(ignore_index),
                              float(softcap) if softcap else 0.0, float(multiplier), red,
                              _ptr(out.loss), _ptr(out.grad_h), _ptr(out.grad_W), _ptr(out.n_correct),
                              stream, dtype, _ptr(workspace), int(workspace.numel()), opts)
    if rc != _lib.FLCE_OK:
        raise _lib.FlceError(rc, "flce_fwd_bwd_ex")
    if check:
        st = _lib.flce_read_status(_ptr(workspace), stream)
        if st != _lib.FLCE_OK:
            raise _lib.FlceError(st, "flce_fwd_bwd_ex (device status)")
    out.grad_h = out.grad_h.reshape(shape)
    if out.loss_rows is not None and reduction == "none":
        out.loss_rows = out.loss_rows.reshape(labels.shape)
    out.workspace = workspace
    out.n_valid = _n_valid_view(workspace)
    return out


def read_status(workspace: torch.Tensor) -> None:
    """Synchronise torch's current stream and raise if the last call that used
    ``workspace`` found a label outside [0, V) that is not ignore_index."""
    stream = torch.cuda.current_stream(workspace.device).cuda_stream
    st = _lib.flce_read_status(_ptr(workspace), stream)
    if st != _lib.FLCE_OK:
        raise _lib.FlceError(st, "device status")


def forward(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100,
            softcap: Optional[float] = None, multiplier: float = 1.0, reduction: str = "mean",
            workspace: Optional[torch.Tensor] = None, check: bool = True,
            row_outputs: bool = False) -> FlceForward:
    """Loss and n_correct only (``flce_fwd``): the cross-entropy-only pass of
    the SpecForge page (Changes), with no gradient and no stored logits."""
    h2, Wc, lab = _prepare(h, W, labels, reduction)
    N, H = h2.shape
    V = Wc.shape[0]
    dtype = _DTYPES[h.dtype]
    ws_bytes = _lib.flce_fwd_workspace_size(N, H, V, dtype, 0)
    if ws_bytes == 0:
        raise _lib.FlceError(_lib.FLCE_EUNSUPPORTED, "flce_fwd_workspace_size")
    dev = h.device
    workspace = _workspace(workspace, ws_bytes, dev)
    loss_rows, lse_rows, pred_rows = _row_buffers(N, dev, reduction == "none", row_outputs)
    res = FlceForward(loss=torch.empty((), dtype=torch.float32, device=dev),
                      n_correct=torch.empty((), dtype=torch.int64, device=dev), workspace=workspace,
                      loss_rows=loss_rows, lse_rows=lse_rows, pred_rows=pred_rows)
    opts = _lib.flce_options_t(loss_rows=_ptr(loss_rows), lse_rows=_ptr(lse_rows), pred_rows=_ptr(pred_rows))
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _lib.flce_fwd(_ptr(h2), _ptr(Wc), _ptr(lab), N, H, V, int(ignore_index),
                       float(softcap) if softcap else 0.0, float(multiplier), _REDUCTIONS[reduction],
                       _ptr(res.loss), _ptr(res.n_correct), stream, dtype, _ptr(workspace),
                       int(workspace.numel()), opts)
    if rc != _lib.FLCE_OK:
        raise _lib.FlceError(rc, "flce_fwd")
    if check:
        st = _lib.flce_read_status(_ptr(workspace), stream)
        if st != _lib.FLCE_OK:
            raise _lib.FlceError(st, "flce_fwd (device status)")
    if reduction == "none":
        res.loss_rows = res.loss_rows.reshape(labels.shape)
    res.n_valid = _n_valid_view(workspace)
    return res


def _padded_cols(V: int, dtype: torch.dtype) -> int:
    per = 16 // torch.tensor([], dtype=dtype).element_size()
    return (V + per - 1) // per * per


def logits(h: torch.Tensor, W: torch.Tensor, softcap: Optional[float] = None, multiplier: float = 1.0,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Materialised logits z = cap(m h W^T) (``flce_logits``), [..., V] in
    the dtype of h.  The rows of the returned tensor have a stride padded to
    16 bytes (a view of a [N, ld] buffer) when V is not a multiple of 8 (bf16)
    or 4 (fp32)."""
    if h.dtype not in _DTYPES or W.dtype != h.dtype:
        raise TypeError(f"h and W must both be bfloat16 or float32 (got {h.dtype}, {W.dtype})")
    H = h.shape[-1]
    h2 = h.reshape(-1, H).contiguous()
    Wc = W.contiguous()
    N, V = h2.shape[0], Wc.shape[0]
    ld = _padded_cols(V, h.dtype)
    if out is None:
        out = torch.empty((N, ld), dtype=h.dtype, device=h.device)
    if out.shape[0] != N or out.stride(1) != 1 or out.stride(0) < V:
        raise ValueError("out must be [N, ld >= V] with unit column stride")
    stream = torch.cuda.current_stream(h.device).cuda_stream
    rc = _lib.flce_logits(_ptr(h2), _ptr(Wc), N, H, V, float(softcap) if softcap else 0.0, float(multiplier),
                          _ptr(out), out.stride(0), stream, _DTYPES[h.dtype])
    if rc != _lib.FLCE_OK:
        raise _lib.FlceError(rc, "flce_logits")
    return out[:, :V].reshape(*h.shape[:-1], V)


@dataclasses.dataclass
class CrossEntropyOutputs:
    loss: torch.Tensor
    n_correct: torch.Tensor
    workspace: torch.Tensor
    grad_logits: Optional[torch.Tensor] = None
    loss_rows: Optional[torch.Tensor] = None
    lse_rows: Optional[torch.Tensor] = None
    pred_rows: Optional[torch.Tensor] = None


def cross_entropy(z: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100, reduction: str = "mean",
                  grad: bool = False, in_place: bool = False, grad_rows: Optional[torch.Tensor] = None,
                  grad_scale: Optional[float] = None, row_outputs: bool = False,
                  check: bool = True) -> CrossEntropyOutputs:
    """Cross-entropy of given logits ``z`` [N, V] (``flce_cross_entropy``),
    optionally with d loss / d z (written into z itself with ``in_place``).
    z may be a row-padded view (row stride a multiple of 16 bytes)."""
    if z.dim() != 2 or z.stride(1) != 1 or z.dtype not in _DTYPES:
        raise ValueError("z must be a [N, V] bfloat16 / float32 tensor with unit column stride")
    if reduction not in _REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    N, V = z.shape
    lab = labels.reshape(-1).to(torch.int64).contiguous()
    dev = z.device
    ws_bytes = _lib.flce_cross_entropy_workspace_size(N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    res = CrossEntropyOutputs(loss=torch.empty((), dtype=torch.float32, device=dev),
                              n_correct=torch.empty((), dtype=torch.int64, device=dev), workspace=ws)
    g = None
    if grad:
        g = z if in_place else torch.empty((N, z.stride(0)), dtype=z.dtype, device=dev)
        res.grad_logits = g if in_place else g[:, :V]
    want_rows = row_outputs or reduction == "none"
    res.loss_rows, res.lse_rows, res.pred_rows = _row_buffers(N, dev, want_rows, want_rows)
    gr = None
    if grad_rows is not None:
        gr = grad_rows.reshape(-1).to(device=dev, dtype=torch.float32).contiguous()
    opts = _lib.flce_options_t(loss_rows=_ptr(res.loss_rows), lse_rows=_ptr(res.lse_rows),
                               pred_rows=_ptr(res.pred_rows), grad_rows=_ptr(gr),
                               grad_scale=float(grad_scale) if grad_scale is not None else 0.0,
                               use_grad_scale=0 if grad_scale is None else 1)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _lib.flce_cross_entropy(_ptr(z), z.stride(0), _ptr(lab), N, V, int(ignore_index), _REDUCTIONS[reduction],
                                 _ptr(res.loss), _ptr(res.n_correct), _ptr(g), g.stride(0) if g is not None else 0,
                                 stream, _DTYPES[z.dtype], _ptr(ws), ws_bytes, opts)
    if rc != _lib.FLCE_OK:
        raise _lib.FlceError(rc, "flce_cross_entropy")
    if check:
        st = _lib.flce_read_status(_ptr(ws), stream)
        if st != _lib.FLCE_OK:
            raise _lib.FlceError(st, "flce_cross_entropy (device status)")
    return res


def scale_grads(g: torch.Tensor, grad_h: Optional[torch.Tensor], grad_W: Optional[torch.Tensor],
                w_dtype: torch.dtype):
    """``flce_scale_grads``: returns (grad_h * g, grad_W * g in ``w_dtype``) as
    new tensors (None where the input is None), g an fp32 scalar that stays on
    the device; one read and one write of each gradient."""
    dev = g.device
    g32 = g.detach().reshape(1).to(torch.float32).contiguous()
    gh_out = torch.empty_like(grad_h) if grad_h is not None else None
    gW_out = torch.empty(grad_W.shape, dtype=w_dtype, device=dev) if grad_W is not None else None
    n_h = grad_h.numel() if grad_h is not None else 0
    n_W = grad_W.numel() if grad_W is not None else 0
    rc = _lib.flce_scale_grads(_ptr(g32), _ptr(grad_h) if n_h else None, _ptr(gh_out) if n_h else None, n_h,
                               _DTYPES[grad_h.dtype] if grad_h is not None else _lib.FLCE_DTYPE_F32,
                               _ptr(grad_W) if n_W else None, _ptr(gW_out) if n_W else None, n_W,
                               _DTYPES[w_dtype], torch.cuda.current_stream(dev).cuda_stream)
    if rc != _lib.FLCE_OK:
        raise _lib.FlceError(rc, "flce_scale_grads")
    return gh_out, gW_out


class _LinearCrossEntropy(torch.autograd.Function):
    """mean / sum: the gradients come out of the fused forward call; backward
    scales them by the upstream scalar on the device (``flce_scale_grads``).
    none: the forward computes the row losses only; backward recomputes the
    logits with the upstream row gradients (grad_W mixes rows, so it cannot be
    rescaled afterwards).  When neither h nor W needs a gradient the forward
    is ``flce_fwd`` (no gradient GEMMs, no [V, H] accumulator).  Nothing here
    synchronises unless ``check`` is set."""

    @staticmethod
    def forward(ctx, h, W, labels, ignore_index, softcap, multiplier, reduction, workspace, check):
        ctx.w_dtype = W.dtype
        ctx.reduction = reduction
        ctx.h_shape = h.shape
        need = ctx.needs_input_grad[:2]
        if reduction == "none" or not any(need):
            o = forward(h.detach(), W.detach(), labels, ignore_index, softcap, multiplier, reduction,
                        workspace=workspace, check=check)
            if reduction == "none" and any(need):
                ctx.save_for_backward(h.detach(), W.detach(), labels)
                ctx.args = (ignore_index, softcap, multiplier, workspace)
            loss = o.loss_rows if reduction == "none" else o.loss
            return loss, o.n_correct
        o = fwd_bwd(h.detach(), W.detach(), labels, ignore_index, softcap, multiplier, reduction,
                    workspace=workspace, check=check)
        ctx.save_for_backward(o.grad_h, o.grad_W)
        return o.loss, o.n_correct

    @staticmethod
    def backward(ctx, grad_loss, _grad_n_correct):
        need_h, need_W = ctx.needs_input_grad[:2]
        if ctx.reduction == "none":
            h, W, labels = ctx.saved_tensors
            ignore_index, softcap, multiplier, workspace = ctx.args
            o = fwd_bwd(h, W, labels, ignore_index, softcap, multiplier, "none", workspace=workspace,
                        check=False, grad_rows=grad_loss.reshape(-1))
            gW = o.grad_W.to(ctx.w_dtype) if need_W else None
            return (o.grad_h if need_h else None), gW, None, None, None, None, None, None, None
        gh, gW = ctx.saved_tensors
        gh_out, gW_out = scale_grads(grad_loss, gh if need_h else None, gW if need_W else None, ctx.w_dtype)
        return gh_out, gW_out, None, None, None, None, None, None, None


def linear_cross_entropy(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                         ignore_index: int = -100, softcap: Optional[float] = None,
                         multiplier: float = 1.0, reduction: str = "mean",
                         workspace: Optional[torch.Tensor] = None, check: bool = False):
    """Differentiable FLCE: returns (loss, n_correct); token accuracy is
    n_correct / number of non-ignored labels (Muse Glimmer page, Summary
    item 2).  With reduction "none" the loss has the shape of ``labels``.

    Nothing synchronises the host by default: out-of-range labels are
    reported by ``read_status(workspace)`` on a caller-owned ``workspace``
    (uint8, reused across steps), or at once with ``check=True``."""
    return _LinearCrossEntropy.apply(h, W, labels, ignore_index, softcap, multiplier, reduction, workspace, check)
