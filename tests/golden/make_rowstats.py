"""Write the oracle's per-row quantities for the full-size workloads.

For each bf16 lm_head workload (c2..c5 in ``synth.CONFIGS``) this regenerates
the seeded inputs, runs ``oracle.row_stats`` over every row in float64, and
stores, per row: log-sum-exp, row max, the label's logit, argmax and top-2
margin, plus the reduced loss.  The GPU parity tests compare against these
(the loss and n_correct need every row; the sampled grad_W rows need every
row's log-sum-exp), and recompute the cheap row-local quantities live.

Only ``oracle`` and ``synth`` are called.  Run from the repository root:
    python tests/golden/make_rowstats.py c2 c3 c4 c5
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402


def path_for(name: str) -> str:
    return os.path.join(HERE, f"{name}_rowstats.npz")


def make(name: str) -> None:
    cfg = synth.CONFIGS[name]
    t0 = time.time()
    case = synth.make_case(cfg)
    W64 = case.W_f32().astype(np.float64)
    h64 = case.h_f32().astype(np.float64)
    print(f"[{name}] inputs {time.time() - t0:.1f}s digest {case.digest()}", flush=True)
    st = oracle.row_stats(h64, W64, case.labels, synth.IGNORE_INDEX, cfg.softcap_T,
                          cfg.multiplier, block=256)
    valid = st["valid"]
    n_valid = int(valid.sum())
    s = oracle.reduction_scale(n_valid, cfg.reduction)
    loss = s * float(st["loss_rows"].sum())
    np.savez(path_for(name), digest=np.array(case.digest()), lse=st["lse"], M=st["M"],
             z_label=st["z_label"], pred=st["pred"].astype(np.int32), margin=st["margin"],
             loss=np.array(loss), n_valid=np.array(n_valid))
    print(f"[{name}] done {time.time() - t0:.1f}s loss {loss:.10g} n_valid {n_valid}", flush=True)


if __name__ == "__main__":
    for n in sys.argv[1:] or ["c2", "c3", "c4", "c5"]:
        make(n)
