"""Helpers for the GPU tests: move seeded inputs to the device, call the HIP
path through the C ABI, and measure errors against the oracle."""
from __future__ import annotations

import sys

import numpy as np

import synth


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(case: synth.Case):
    import torch
    dev = torch.device("cuda", 0)
    if case.cfg.dtype == "bf16":
        h = torch.from_numpy(case.h.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(case.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        h = torch.from_numpy(case.h).to(dev)
        W = torch.from_numpy(case.W).to(dev)
    labels = torch.from_numpy(case.labels).to(dev)
    return h, W, labels


def run_case(case: synth.Case, h=None, W=None, labels=None, **kw):
    """One flce_fwd_bwd call (through the ctypes binding of the C ABI)."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    if h is None:
        h, W, labels = to_device(case)
    cfg = case.cfg
    o = L.fwd_bwd(h, W, labels, ignore_index=kw.get("ignore_index", synth.IGNORE_INDEX),
                  softcap=cfg.softcap_T if cfg.softcap_T > 0 else None,
                  multiplier=cfg.multiplier, reduction=cfg.reduction)
    torch.cuda.synchronize()
    return o


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def tolerances(dtype: str):
    """Loss relative error and gradient relative Frobenius error bounds."""
    return (1e-5, 1e-4) if dtype == "f32" else (2e-3, 2e-2)
