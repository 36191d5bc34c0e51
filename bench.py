#!/usr/bin/env python3
"""Throughput of fused linear cross-entropy forward+backward on one MI355X.

One step = one ``flce_fwd_bwd`` call over the whole batch: logits GEMM with the
fused softcap / log-sum-exp / argmax epilogue, row merge, grad logits, the
grad_h and grad_W GEMMs, for every token chunk, and the loss/n_correct
finalisation.  Inputs are seeded synthetic tensors (``synth``) already resident
in HBM when the timed region starts.

Prints one JSON line (rank 0) with the metric, a roofline entry for the
dominant kernel (its average launch duration measured with HIP events on its
own stream during the timed steps), every kernel's time per step (each GEMM
also as TFLOP/s and fraction of the dense peak) and the fp64 oracle timed on
a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FLCE fwd+bwd tokens/sec at V=202048,H=6656 bf16; % of MFMA bf16 peak"
METRIC_FWD = "FLCE forward-only tokens/sec at V=202048,H=6656 bf16; % of MFMA bf16 peak"
METRIC_MAT = "materialised logits + cross-entropy forward tokens/sec at V=202048,H=6656 bf16; % of MFMA bf16 peak"
# MI355X dense MFMA peaks (TFLOP/s).
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
GEMM_KINDS = ("fwd_logits", "grad_h", "grad_W", "logits")

WORKLOAD_TEXT = {
    "c1": "fp32 small: N=256, H=128, V=1024, 10% ignore_index, mean",
    "c2": "bf16 lm_head: N=4096, H=4096, V=128256, 5% ignore_index, mean",
    "c3": "bf16 DeepSeek-V3-shaped lm_head: N=8192, H=7168, V=129280, Zipf(1.1) labels, 5% ignore_index, mean",
    "c4": "bf16 Muse-Glimmer-shaped lm_head: N=8192, H=6656, V=202048, softcap T=30, multiplier 0.5, "
          "uniform labels, 5% ignore_index, mean, n_correct",
    "c5": "bf16 long context: N=32768 (4 x 8192), H=7168, V=129280, softcap T=30, Zipf(1.1) labels, "
          "20% ignore_index as tail padding, sum",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "linear_cross_entropy_gemm_amd", "csrc")
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    """Hash of the sources that decide HBM traffic (the kernels and the
    chunk / split planner; not the argument checks or the timing facility): a
    traffic figure measured on other kernels or launch plans is stale."""
    m = hashlib.sha256()
    files = [f for f in glob.glob(os.path.join(CSRC, "*"))
             if f.endswith((".hip", ".hpp")) or os.path.basename(f) == "flce_plan.cpp"]
    for f in sorted(files):
        m.update(os.path.basename(f).encode())
        m.update(open(f, "rb").read())
    return m.hexdigest()[:16]


def copy_calibration() -> int:
    """A plain device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES),
    three times: the reference the FETCH_SIZE / WRITE_SIZE counters are
    scaled by."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {COPY_BYTES} bytes x3")
    return 0


def _pmc_per_dispatch(d: str, counter: str, name_part: str) -> list:
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    return vals


def summarize_traffic(kernel: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                      copy_write_dir: str, out: str, command: str) -> int:
    """Turn four rocprofv3 --pmc runs into HBM bytes per launch of `kernel`."""
    cf = _pmc_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copy")
    cw = _pmc_per_dispatch(copy_write_dir, "WRITE_SIZE", "copy")
    # "grad_h" must not also match grad_h_reduce_kernel
    kf = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE", kernel + "_kernel")
    kw = _pmc_per_dispatch(write_dir, "WRITE_SIZE", kernel + "_kernel")
    if not (cf and cw and kf and kw):
        log("[bench] missing counter values")
        return 1
    # counters read in KiB; the factor maps them onto the copy's known bytes
    f_scale = COPY_BYTES / (max(cf) * 1024.0)
    w_scale = COPY_BYTES / (max(cw) * 1024.0)
    fetch = sum(kf) / len(kf) * 1024.0 * f_scale
    write = sum(kw) / len(kw) * 1024.0 * w_scale
    rec = {"kernel": kernel, "source_hash": kernel_source_hash(), "launches": len(kf),
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "traffic_bytes_per_launch": fetch + write,
           "copy_fetch_kib": max(cf), "copy_write_kib": max(cw), "fetch_scale": f_scale, "write_scale": w_scale,
           "command": command}
    json.dump(rec, open(out, "w"), indent=1)
    log(f"[bench] {kernel}: fetch {fetch / 1e9:.3f} GB + write {write / 1e9:.3f} GB per launch -> {out}")
    return 0


def stored_traffic(kernel: str, config: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{config}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec["traffic_bytes_per_launch"]


def blas_threads() -> int:
    try:
        import numpy  # noqa: F401
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_vendor() -> str:
    """numpy's BLAS library as threadpoolctl reports it (internal_api and
    version)."""
    try:
        import numpy  # noqa: F401  (loads the BLAS threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            p = libs[0]
            return f"{p.get('internal_api', 'unknown')} {p.get('version') or ''}".strip()
    except Exception:
        pass
    return "unknown"


def host_record() -> dict:
    return {"cores": blas_threads(), "cpu_model": cpu_model(), "blas": blas_vendor(),
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(case, n_tokens: int) -> dict:
    """The fp64 oracle, as it stands, on the first n_tokens rows of the same
    inputs: full forward and backward for those rows."""
    import oracle
    import synth
    cfg = case.cfg
    n = min(n_tokens, cfg.N)
    h = case.h_f32()[:n]
    W = case.W_f32()
    lab = case.labels[:n]
    t0 = time.perf_counter()
    oracle.flce_reference(h, W, lab, synth.IGNORE_INDEX, cfg.softcap_T, cfg.multiplier, cfg.reduction)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", **host_record(), "kind": "oracle",
            "sample": f"first {n} of {cfg.N} tokens of the same seeded inputs, full fp64 forward+backward "
                      f"(loss, argmax, grad_h rows, the sample's [V,H] grad_W) in {dt:.1f} s"}


def cpu_baseline_forward(case, n_tokens: int) -> dict:
    """The fp64 oracle's forward (row statistics over the full vocabulary) on
    the first n_tokens rows of the same inputs."""
    import oracle
    import synth
    cfg = case.cfg
    n = min(n_tokens, cfg.N)
    t0 = time.perf_counter()
    oracle.row_stats(case.h_f32()[:n], case.W_f32(), case.labels[:n], synth.IGNORE_INDEX, cfg.softcap_T,
                     cfg.multiplier)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", **host_record(), "kind": "oracle",
            "sample": f"first {n} of {cfg.N} tokens of the same seeded inputs, fp64 forward "
                      f"(log-sum-exp, label logit, argmax per row) in {dt:.1f} s"}


def time_calls(call, stream, steps: int, warmup: int):
    """warmup untimed calls, then `steps` timed ones between synchronizations,
    with the library's per-kernel event timing on."""
    import torch
    import linear_cross_entropy_gemm_amd as L
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    L.flce_profile_enable(True)
    L.flce_profile_read(stream.cuda_stream, reset=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    prof = L.flce_profile_read(stream.cuda_stream, reset=True)
    L.flce_profile_enable(False)
    return ev0.elapsed_time(ev1) / steps, prof


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--cpu-tokens", type=int, default=1536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=6,
                    metavar=("KERNEL", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "OUT"),
                    help="write HBM traffic per launch from four rocprofv3 --pmc runs")
    ap.add_argument("--command", default="", help="command text recorded with --summarize-traffic")
    ap.add_argument("--entry", default="fwd_bwd", choices=("fwd_bwd", "fwd", "materialised"),
                    help="fwd_bwd (default): flce_fwd_bwd, the headline metric; fwd: the forward-only "
                         "flce_fwd (loss and n_correct, 2*N*H*V); materialised: flce_logits into an "
                         "[N, V] buffer then flce_cross_entropy (the non-fused forward)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic, command=args.command)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not part of this build", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import linear_cross_entropy_gemm_amd as L
    import synth

    cfg = synth.CONFIGS[args.config]
    t0 = time.perf_counter()
    log(f"[bench] generating {args.config} inputs ...")
    case = synth.make_case(cfg)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if cfg.dtype == "bf16":
        h = torch.from_numpy(case.h.view(np.int16)).to(dev).view(torch.bfloat16)
        W = torch.from_numpy(case.W.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        h = torch.from_numpy(case.h).to(dev)
        W = torch.from_numpy(case.W).to(dev)
    lab = torch.from_numpy(case.labels).to(dev)
    softcap = cfg.softcap_T if cfg.softcap_T > 0 else None
    kw = dict(softcap=softcap, multiplier=cfg.multiplier, reduction=cfg.reduction)
    dtype_code = L.FLCE_DTYPE_BF16 if cfg.dtype == "bf16" else L.FLCE_DTYPE_F32
    plan = L.flce_plan(cfg.N, cfg.H, cfg.V, dtype_code)
    log(f"[bench] plan {plan.as_dict()}")

    stream = torch.cuda.current_stream(dev)
    fwd_only = args.entry in ("fwd", "materialised")
    memory = None
    red = {"mean": L.FLCE_REDUCTION_MEAN, "sum": L.FLCE_REDUCTION_SUM}[cfg.reduction]
    if args.entry == "materialised":
        z = L.logits(h, W, softcap, cfg.multiplier)
        ce = L.cross_entropy(z, lab, synth.IGNORE_INDEX, cfg.reduction)
        zbase = z.as_strided((cfg.N, z.stride(0)), (z.stride(0), 1))
        ws = ce.workspace
        raw_z = (h.data_ptr(), W.data_ptr(), cfg.N, cfg.H, cfg.V, float(softcap or 0.0), float(cfg.multiplier),
                 z.data_ptr(), z.stride(0), stream.cuda_stream, dtype_code)
        raw_ce = (z.data_ptr(), z.stride(0), lab.data_ptr(), cfg.N, cfg.V, synth.IGNORE_INDEX, red,
                  ce.loss.data_ptr(), ce.n_correct.data_ptr(), None, 0, stream.cuda_stream, dtype_code,
                  ws.data_ptr(), ws.numel(), None)

        def call():
            rc = L.flce_logits(*raw_z)
            if rc == L.FLCE_OK:
                rc = L.flce_cross_entropy(*raw_ce)
            if rc != L.FLCE_OK:
                raise L.FlceError(rc, "materialised path")
        loss_t, nc_t = ce.loss, ce.n_correct
        memory = {"logits_bytes": zbase.numel() * zbase.element_size(), "workspace_bytes": ws.numel(),
                  "fused_forward_workspace_bytes": L.flce_fwd_workspace_size(cfg.N, cfg.H, cfg.V, dtype_code)}
    elif fwd_only:
        f = L.forward(h, W, lab, **kw)                  # allocates outputs + workspace, checks status
        ws = f.workspace
        raw = (h.data_ptr(), W.data_ptr(), lab.data_ptr(), cfg.N, cfg.H, cfg.V, synth.IGNORE_INDEX,
               float(softcap or 0.0), float(cfg.multiplier), red, f.loss.data_ptr(), f.n_correct.data_ptr(),
               stream.cuda_stream, dtype_code, ws.data_ptr(), ws.numel(), None)

        def call():
            rc = L.flce_fwd(*raw)
            if rc != L.FLCE_OK:
                raise L.FlceError(rc, "flce_fwd")
        loss_t, nc_t = f.loss, f.n_correct
    else:
        o = L.fwd_bwd(h, W, lab, **kw)                  # allocates outputs + workspace, checks status
        ws = o.workspace

        def call():
            L.fwd_bwd(h, W, lab, workspace=ws, out=o, check=False, **kw)
        loss_t, nc_t = o.loss, o.n_correct
    ms, prof = time_calls(call, stream, args.steps, args.warmup)
    log(f"[bench] {args.entry}: loss {loss_t.item():.6f} n_correct {nc_t.item()}")
    st = L.flce_read_status(ws.data_ptr(), stream.cuda_stream)
    if st != L.FLCE_OK:
        raise L.FlceError(st, "device status after timing")
    tok_s = cfg.N / (ms * 1e-3)
    n_gemm = 1 if fwd_only else 3
    flops = 2.0 * n_gemm * cfg.N * cfg.H * cfg.V
    flops_valid = 2.0 * n_gemm * cfg.n_valid * cfg.H * cfg.V
    peak = PEAK_TFLOPS[cfg.dtype]
    pct = flops / (ms * 1e-3) / (peak * 1e12) * 100.0
    pct_valid = flops_valid / (ms * 1e-3) / (peak * 1e12) * 100.0
    basis = "2NHV" if fwd_only else "6NHV"
    log(f"[bench] {ms:.3f} ms/step, {tok_s:,.0f} tokens/s, {pct:.1f}% of MFMA peak "
        f"({basis} basis; {pct_valid:.1f}% on N_valid)")

    kernels = {}
    for k, (tot, n) in prof.items():
        if n:
            kernels[k] = {"avg_ms": tot / n, "launches_per_step": n / args.steps,
                          "ms_per_step": tot / args.steps}
            log(f"[bench]   {k:14s} {tot / args.steps:8.3f} ms/step  {n / args.steps:4.1f} launches  "
                f"{tot / n:8.3f} ms avg")
    dom = max((k for k in kernels if k in GEMM_KINDS), key=lambda k: kernels[k]["ms_per_step"])
    # The fused entries pack the valid rows before the GEMMs, so their GEMM
    # launches together process N_valid token rows; the materialised logits
    # GEMM processes all N.
    rows_alg = cfg.n_valid if args.entry in ("fwd_bwd", "fwd") else cfg.N
    for k in kernels:
        if k in GEMM_KINDS:   # every GEMM does 2 * rows * H * V per step over its launches
            tf = 2.0 * rows_alg * cfg.H * cfg.V / (kernels[k]["ms_per_step"] * 1e-3) / 1e12
            kernels[k]["tflops"] = tf
            kernels[k]["frac_of_peak"] = tf / peak
    flops_per_launch = 2.0 * rows_alg * cfg.H * cfg.V / kernels[dom]["launches_per_step"]
    achieved = flops_per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
    traffic = stored_traffic(dom, args.config)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "flops_per_launch": flops_per_launch, "token_rows_per_launch": rows_alg / kernels[dom]["launches_per_step"],
                "avg_launch_ms": round(kernels[dom]["avg_ms"], 4)}

    result = {
        "metric": {"fwd": METRIC_FWD, "materialised": METRIC_MAT}.get(args.entry, METRIC),
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config], "name": args.config, "N": cfg.N, "H": cfg.H,
                   "V": cfg.V, "n_valid": cfg.n_valid, "softcap_T": cfg.softcap_T,
                   "multiplier": cfg.multiplier, "reduction": cfg.reduction,
                   "entry": {"fwd": "flce_fwd", "materialised": "flce_logits + flce_cross_entropy"}.get(
                       args.entry, "flce_fwd_bwd"),
                   "chunk_rows": cfg.N if fwd_only else plan.chunk_rows,
                   "n_chunks": 1 if fwd_only else plan.n_chunks, "split_k": plan.split_k,
                   "parallelism": "single GPU"},
        f"pct_peak_{basis}": round(pct, 2), f"pct_peak_{basis.replace('N', 'Nvalid', 1)}": round(pct_valid, 2),
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kernels.items()},
        "roofline": roofline,
    }
    if memory is not None:
        result["memory"] = memory
    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on {args.cpu_tokens} tokens (host cores) ...")
        result["cpu_baseline"] = (cpu_baseline_forward(case, 3 * args.cpu_tokens) if fwd_only
                                  else cpu_baseline(case, args.cpu_tokens))
        log(f"[bench] cpu baseline {result['cpu_baseline']['value']:.1f} tokens/s")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
