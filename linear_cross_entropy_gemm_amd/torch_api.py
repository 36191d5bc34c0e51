"""PyTorch-facing wrappers: device memory and the current stream come from
torch; the whole forward and backward runs in ``flce_fwd_bwd``."""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.FLCE_DTYPE_BF16, torch.float32: _lib.FLCE_DTYPE_F32}
_REDUCTIONS = {"mean": _lib.FLCE_REDUCTION_MEAN, "sum": _lib.FLCE_REDUCTION_SUM}


@dataclasses.dataclass
class FlceOutputs:
    loss: torch.Tensor        # [] fp32
    grad_h: torch.Tensor      # [N, H] dtype of h
    grad_W: torch.Tensor      # [V, H] fp32
    n_correct: torch.Tensor   # [] int64
    workspace: torch.Tensor   # uint8, holds the status word


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def fwd_bwd(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, ignore_index: int = -100,
            softcap: Optional[float] = None, multiplier: float = 1.0, reduction: str = "mean",
            workspace: Optional[torch.Tensor] = None, out: Optional[FlceOutputs] = None,
            check: bool = True) -> FlceOutputs:
    """One call of ``flce_fwd_bwd`` on torch's current stream.

    ``h`` [..., H] is flattened to [N, H] and ``grad_h`` restored to its shape
    (SpecForge PR 1007, Changes: flatten rows for the vocabulary projection,
    then restore the output shape)."""
    if h.dtype not in _DTYPES or W.dtype != h.dtype:
        raise TypeError(f"h and W must both be bfloat16 or float32 (got {h.dtype}, {W.dtype})")
    if not h.is_cuda or not W.is_cuda or not labels.is_cuda:
        raise ValueError("h, W and labels must be on the GPU")
    shape = h.shape
    H = shape[-1]
    h2 = h.reshape(-1, H).contiguous()
    N = h2.shape[0]
    V = W.shape[0]
    Wc = W.contiguous()
    lab = labels.reshape(-1).to(torch.int64).contiguous()
    if lab.numel() != N:
        raise ValueError("labels must have one entry per row of h")
    dtype = _DTYPES[h.dtype]
    red = _REDUCTIONS[reduction]
    ws_bytes = _lib.flce_workspace_size(N, H, V, dtype, 0)
    if ws_bytes == 0:
        raise _lib.FlceError(_lib.FLCE_EUNSUPPORTED, "flce_workspace_size")
    dev = h.device
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if out is None:
        out = FlceOutputs(
            loss=torch.empty((), dtype=torch.float32, device=dev),
            grad_h=torch.empty((N, H), dtype=h.dtype, device=dev),
            grad_W=torch.empty((V, H), dtype=torch.float32, device=dev),
            n_correct=torch.empty((), dtype=torch.int64, device=dev),
            workspace=workspace,
        )
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _lib.flce_fwd_bwd(_ptr(h2), _ptr(Wc), _ptr(lab), N, H, V, int(ignore_index),
                           float(softcap) if softcap else 0.0, float(multiplier), red,
                           _ptr(out.loss), _ptr(out.grad_h), _ptr(out.grad_W), _ptr(out.n_correct),
                           stream, dtype, _ptr(workspace), int(workspace.numel()))
    if rc != _lib.FLCE_OK:
        raise _lib.FlceError(rc, "flce_fwd_bwd")
    if check:
        st = _lib.flce_read_status(_ptr(workspace), stream)
        if st != _lib.FLCE_OK:
            raise _lib.FlceError(st, "flce_fwd_bwd (device status)")
    out.grad_h = out.grad_h.reshape(shape)
    out.workspace = workspace
    return out


class _LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, h, W, labels, ignore_index, softcap, multiplier, reduction):
        o = fwd_bwd(h.detach(), W.detach(), labels, ignore_index, softcap, multiplier, reduction)
        ctx.save_for_backward(o.grad_h, o.grad_W)
        ctx.w_dtype = W.dtype
        return o.loss, o.n_correct

    @staticmethod
    def backward(ctx, grad_loss, _grad_n_correct):
        gh, gW = ctx.saved_tensors
        g = grad_loss.to(torch.float32)
        gh = gh * g.to(gh.dtype)
        gW = (gW * g).to(ctx.w_dtype)
        return gh, gW, None, None, None, None, None


def linear_cross_entropy(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                         ignore_index: int = -100, softcap: Optional[float] = None,
                         multiplier: float = 1.0, reduction: str = "mean"):
    """Differentiable FLCE: returns (loss, n_correct); token accuracy is
    n_correct / number of non-ignored labels (Muse Glimmer page, Summary
    item 2).  The gradients are computed in the forward call and scaled by
    the upstream gradient in backward."""
    return _LinearCrossEntropy.apply(h, W, labels, ignore_index, softcap, multiplier, reduction)
