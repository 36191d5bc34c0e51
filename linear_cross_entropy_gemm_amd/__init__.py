"""MI355X-native fused linear cross-entropy (FLCE).

The lm_head projection of hidden states onto the vocabulary, fused with the
cross-entropy loss, the token-accuracy argmax and the backward pass, without
ever materialising the [tokens, vocab] logits (Liger-Kernel "Muse Glimmer" and
"DeepSeek-V3" commit pages, Summary and Memory sections).  All computation runs
in the HIP kernels of ``libflce.so``; this package only marshals arguments and
uses PyTorch for device memory and streams.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    EXPORTED,
    FLCE_DTYPE_BF16,
    FLCE_DTYPE_F32,
    FLCE_EDEVICE,
    FLCE_EINVAL,
    FLCE_ELABEL,
    FLCE_ESCRATCH,
    FLCE_EUNSUPPORTED,
    FLCE_EWORKSPACE,
    FLCE_OK,
    FLCE_REDUCTION_MEAN,
    FLCE_REDUCTION_NONE,
    FLCE_REDUCTION_SUM,
    KERNEL_KINDS,
    NOALLOC_SCRATCH_BYTES,
    WS_N_VALID_OFFSET,
    FlceError,
    flce_cross_entropy,
    flce_cross_entropy_workspace_size,
    flce_fwd,
    flce_fwd_bwd,
    flce_fwd_bwd_ex,
    flce_fwd_bwd_noalloc,
    flce_fwd_workspace_size,
    flce_logits,
    flce_options_t,
    flce_profile_enable,
    flce_profile_read,
    flce_plan,
    flce_read_status,
    flce_scale_grads,
    flce_strerror,
    flce_workspace_size,
)
from .torch_api import (  # noqa: F401
    CrossEntropyOutputs,
    FlceForward,
    FlceOutputs,
    cross_entropy,
    forward,
    fwd_bwd,
    linear_cross_entropy,
    logits,
    read_status,
    scale_grads,
    token_accuracy,
)
