"""ctypes binding of ``libflce.so`` -- argument marshalling only.

Each function here has the name and arguments of the C ABI declared in
``include/flce.h``; every step of the computation runs in the library's HIP
kernels.  Importing this module fails loudly when the library is missing: there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflce.so")

FLCE_DTYPE_BF16 = 0
FLCE_DTYPE_F32 = 1
FLCE_REDUCTION_MEAN = 0
FLCE_REDUCTION_SUM = 1
FLCE_REDUCTION_NONE = 2

FLCE_OK = 0
FLCE_EINVAL = 1
FLCE_EWORKSPACE = 2
FLCE_EDEVICE = 3
FLCE_ELABEL = 4
FLCE_EUNSUPPORTED = 5
FLCE_ESCRATCH = 6

# Byte offset of N_valid (uint64) in a workspace after a call (FLCE_WS_N_VALID_OFFSET).
WS_N_VALID_OFFSET = 8

# Static scratch of flce_fwd_bwd_noalloc (FLCE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 256 << 20

# Every symbol include/flce.h declares.
EXPORTED = ("flce_plan", "flce_workspace_size", "flce_fwd_bwd", "flce_fwd_bwd_ex", "flce_fwd_bwd_noalloc",
            "flce_fwd_workspace_size",
            "flce_fwd", "flce_logits", "flce_cross_entropy_workspace_size", "flce_cross_entropy",
            "flce_scale_grads", "flce_read_status", "flce_strerror", "flce_profile_enable", "flce_profile_read")

# Kernel kinds of the per-kernel timing facility (index order of the arrays).
KERNEL_KINDS = ("label_scan", "fwd_logits", "row_merge", "grad_logits", "grad_h", "grad_h_reduce",
                "grad_W", "finalize", "zero", "logits", "cross_entropy", "scale")


class flce_plan_t(ctypes.Structure):
    _fields_ = [
        ("chunk_rows", ctypes.c_int64),
        ("n_chunks", ctypes.c_int64),
        ("vocab_padded", ctypes.c_int64),
        ("split_k", ctypes.c_int64),
        ("logits_chunk_bytes", ctypes.c_size_t),
        ("workspace_bytes", ctypes.c_size_t),
        ("grad_W_bytes", ctypes.c_size_t),
    ]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class flce_options_t(ctypes.Structure):
    """Options of flce_fwd_bwd_ex / flce_fwd (device addresses as ints, 0 = none)."""
    _fields_ = [
        ("loss_rows", ctypes.c_void_p),
        ("lse_rows", ctypes.c_void_p),
        ("pred_rows", ctypes.c_void_p),
        ("grad_rows", ctypes.c_void_p),
        ("grad_scale", ctypes.c_float),
        ("accumulate_grad_W", ctypes.c_int),
        ("use_grad_scale", ctypes.c_int),
    ]


class FlceError(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        self.code = code
        super().__init__(f"{where}: FLCE error {code}: {flce_strerror(code)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python linear_cross_entropy_gemm_amd/build.py` "
            "(the FLCE path has no fallback implementation)")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7.  If
    # this library were loaded first, the dynamic linker would map the system
    # ROCm runtime for it and torch would then load its own second copy;
    # device pointers and streams of one runtime are not valid in the other,
    # and every launch fails.  Loading torch first makes this library bind to
    # torch's runtime (same soname).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i64, sz, vp, i32, f32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.flce_plan.argtypes = [i64, i64, i64, i32, sz, ctypes.POINTER(flce_plan_t)]
    lib.flce_plan.restype = i32
    lib.flce_workspace_size.argtypes = [i64, i64, i64, i32, sz]
    lib.flce_workspace_size.restype = sz
    lib.flce_fwd_bwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, f32, i32,
                                 vp, vp, vp, vp, vp, i32, vp, sz]
    lib.flce_fwd_bwd.restype = i32
    lib.flce_fwd_bwd_ex.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, f32, i32,
                                    vp, vp, vp, vp, vp, i32, vp, sz, ctypes.POINTER(flce_options_t)]
    lib.flce_fwd_bwd_ex.restype = i32
    lib.flce_fwd_bwd_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, f32, i32,
                                         vp, vp, vp, vp, vp, vp, i32, ctypes.POINTER(flce_options_t)]
    lib.flce_fwd_bwd_noalloc.restype = i32
    lib.flce_fwd_workspace_size.argtypes = [i64, i64, i64, i32, sz]
    lib.flce_fwd_workspace_size.restype = sz
    lib.flce_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, f32, i32,
                             vp, vp, vp, i32, vp, sz, ctypes.POINTER(flce_options_t)]
    lib.flce_fwd.restype = i32
    lib.flce_logits.argtypes = [vp, vp, i64, i64, i64, f32, f32, vp, i64, vp, i32]
    lib.flce_logits.restype = i32
    lib.flce_cross_entropy_workspace_size.argtypes = [i64]
    lib.flce_cross_entropy_workspace_size.restype = sz
    lib.flce_cross_entropy.argtypes = [vp, i64, vp, i64, i64, i64, i32, vp, vp, vp, i64, vp, i32, vp, sz,
                                       ctypes.POINTER(flce_options_t)]
    lib.flce_cross_entropy.restype = i32
    lib.flce_scale_grads.argtypes = [vp, vp, vp, i64, i32, vp, vp, i64, i32, vp]
    lib.flce_scale_grads.restype = i32
    lib.flce_read_status.argtypes = [vp, vp]
    lib.flce_read_status.restype = i32
    lib.flce_strerror.argtypes = [i32]
    lib.flce_strerror.restype = ctypes.c_char_p
    lib.flce_profile_enable.argtypes = [i32]
    lib.flce_profile_enable.restype = i32
    lib.flce_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), i32]
    lib.flce_profile_read.restype = i32
    return lib


_lib = _load()


def flce_plan(N: int, H: int, V: int, dtype: int, budget_bytes: int = 0) -> flce_plan_t:
    out = flce_plan_t()
    rc = _lib.flce_plan(N, H, V, dtype, budget_bytes, ctypes.byref(out))
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_plan")
    return out


def flce_workspace_size(N: int, H: int, V: int, dtype: int, budget_bytes: int = 0) -> int:
    return int(_lib.flce_workspace_size(N, H, V, dtype, budget_bytes))


def flce_fwd_bwd(h: int, W: int, labels: int, N: int, H: int, V: int, ignore_index: int,
                 softcap_T: float, multiplier: float, reduction: int, loss: int, grad_h: int,
                 grad_W: int, n_correct, stream: int, dtype: int, workspace: int,
                 workspace_bytes: int) -> int:
    """Raw call with device addresses as ints; returns the C return code."""
    return int(_lib.flce_fwd_bwd(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier,
                                 reduction, loss, grad_h, grad_W, n_correct, stream, dtype,
                                 workspace, workspace_bytes))


def _opts(options):
    return None if options is None else ctypes.byref(options)


def flce_fwd_bwd_ex(h: int, W: int, labels: int, N: int, H: int, V: int, ignore_index: int,
                    softcap_T: float, multiplier: float, reduction: int, loss: int, grad_h: int,
                    grad_W: int, n_correct, stream: int, dtype: int, workspace: int,
                    workspace_bytes: int, options) -> int:
    """Raw call; ``options`` is a flce_options_t or None.  Returns the C return code."""
    return int(_lib.flce_fwd_bwd_ex(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier,
                                    reduction, loss, grad_h, grad_W, n_correct, stream, dtype,
                                    workspace, workspace_bytes, _opts(options)))


def flce_fwd_bwd_noalloc(h: int, W: int, labels: int, N: int, H: int, V: int, ignore_index: int,
                         softcap_T: float, multiplier: float, reduction: int, loss: int, grad_h: int,
                         grad_W: int, n_correct, status, stream: int, dtype: int, options) -> int:
    """Raw call of the allocation-free variant (static scratch, no workspace
    argument; ``status`` receives the device-side status word).  Returns the
    C return code."""
    return int(_lib.flce_fwd_bwd_noalloc(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier,
                                         reduction, loss, grad_h, grad_W, n_correct, status, stream, dtype,
                                         _opts(options)))


def flce_fwd_workspace_size(N: int, H: int, V: int, dtype: int, budget_bytes: int = 0) -> int:
    return int(_lib.flce_fwd_workspace_size(N, H, V, dtype, budget_bytes))


def flce_fwd(h: int, W: int, labels: int, N: int, H: int, V: int, ignore_index: int,
             softcap_T: float, multiplier: float, reduction: int, loss: int, n_correct, stream: int,
             dtype: int, workspace: int, workspace_bytes: int, options) -> int:
    """Raw forward-only call; returns the C return code."""
    return int(_lib.flce_fwd(h, W, labels, N, H, V, ignore_index, softcap_T, multiplier, reduction,
                             loss, n_correct, stream, dtype, workspace, workspace_bytes, _opts(options)))


def flce_logits(h: int, W: int, N: int, H: int, V: int, softcap_T: float, multiplier: float, logits: int,
                ld_logits: int, stream: int, dtype: int) -> int:
    return int(_lib.flce_logits(h, W, N, H, V, softcap_T, multiplier, logits, ld_logits, stream, dtype))


def flce_cross_entropy_workspace_size(N: int) -> int:
    return int(_lib.flce_cross_entropy_workspace_size(N))


def flce_cross_entropy(logits: int, ld_logits: int, labels: int, N: int, V: int, ignore_index: int,
                       reduction: int, loss: int, n_correct, grad_logits, ld_grad: int, stream: int, dtype: int,
                       workspace: int, workspace_bytes: int, options) -> int:
    return int(_lib.flce_cross_entropy(logits, ld_logits, labels, N, V, ignore_index, reduction, loss,
                                       n_correct, grad_logits, ld_grad, stream, dtype, workspace,
                                       workspace_bytes, _opts(options)))


def flce_scale_grads(grad_scale: int, grad_h_in, grad_h_out, n_h: int, h_dtype: int, grad_W_in, grad_W_out,
                     n_W: int, w_dtype: int, stream: int) -> int:
    """Raw call: grad_h_out = grad_h_in * g and grad_W_out = grad_W_in * g (g at
    device address grad_scale); returns the C return code."""
    return int(_lib.flce_scale_grads(grad_scale, grad_h_in, grad_h_out, n_h, h_dtype, grad_W_in, grad_W_out,
                                     n_W, w_dtype, stream))


def flce_read_status(workspace: int, stream: int) -> int:
    return int(_lib.flce_read_status(workspace, stream))


def flce_strerror(code: int) -> str:
    return _lib.flce_strerror(code).decode()


def flce_profile_enable(on: bool) -> int:
    return int(_lib.flce_profile_enable(1 if on else 0))


def flce_profile_read(stream: int, reset: bool = True) -> dict:
    """{kind: (total_ms, launches)} accumulated since the last reset."""
    n = len(KERNEL_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    rc = _lib.flce_profile_read(stream, ms, cnt, 1 if reset else 0)
    if rc != FLCE_OK:
        raise FlceError(rc, "flce_profile_read")
    return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNEL_KINDS)}


def lib_handle() -> ctypes.CDLL:
    return _lib
