"""Independent calls on separate streams: the library keeps no per-call state
outside the caller's workspace and outputs, so two calls enqueued on two
streams (each with its own workspace) may run at the same time and must give
bitwise the results each gives alone (the kernels are deterministic), with
valid-row packing and without it.  The streams keep the default priority."""
import numpy as np
import pytest

import synth
from gpu_util import log, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]

IGN = synth.IGNORE_INDEX


def _case(base, N, H, V, T, m, red, seed):
    cfg = synth.small_config(base, softcap_T=T, multiplier=m, reduction=red)
    return synth.make_case(cfg, N=N, H=H, V=V, seed=seed)


def _call(L, inputs, case, rows):
    h, W, lab = inputs
    T = case.cfg.softcap_T
    return L.fwd_bwd(h, W, lab, IGN, T if T > 0 else None, case.cfg.multiplier, case.cfg.reduction,
                     check=False, row_outputs=rows)


def _host(o):
    """The outputs' bits on the host (bf16 as int16: numpy has no bfloat16)."""
    import torch
    out = {}
    for k in ("loss", "n_correct", "grad_h", "grad_W", "lse_rows", "pred_rows"):
        t = getattr(o, k)
        if t is None:
            continue
        out[k] = (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy().copy()
    return out


@pytest.mark.parametrize("rows", [False, True], ids=["packed", "row_outputs"])
def test_two_streams_match_separate_calls(rows):
    import torch
    import linear_cross_entropy_gemm_amd as L
    cases = [_case("c4", 700, 256, 3000, 30.0, 0.5, "mean", 11), _case("c2", 513, 320, 2100, 0.0, 1.0, "sum", 12)]
    inputs = [to_device(c) for c in cases]
    log(f"[streams] two cases, each alone on the current stream (row outputs {rows})")
    alone = []
    for c, x in zip(cases, inputs):
        o = _call(L, x, c, rows)
        torch.cuda.synchronize()
        alone.append(_host(o))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        log(f"[streams] both cases enqueued on two streams, repetition {rep}")
        outs = [None, None]
        torch.cuda.synchronize()
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                outs[i] = _call(L, inputs[i], cases[i], rows)
        torch.cuda.synchronize()
        for i in (0, 1):
            got = _host(outs[i])
            for k, ref in alone[i].items():
                assert np.array_equal(got[k], ref), (rep, i, k)
