"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, plans chunks as documented and rejects bad arguments before touching
the GPU (no compute call runs here)."""
import ctypes
import json
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = pytest.importorskip("linear_cross_entropy_gemm_amd")


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "flce.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    decl = declared_symbols()
    assert decl == sorted(L.EXPORTED)
    lib = ctypes.CDLL(L._lib.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name


def test_kernel_kinds_match_the_header():
    import re
    text = open(os.path.join(ROOT, "include", "flce.h")).read()
    kinds = dict((name.lower(), int(v)) for name, v in re.findall(r"FLCE_KERNEL_(\w+)\s*=\s*(\d+)", text))
    n = kinds.pop("kinds")
    assert n == len(L.KERNEL_KINDS)
    assert [k for k, _ in sorted(kinds.items(), key=lambda kv: kv[1])] == [k.lower() for k in L.KERNEL_KINDS]


def test_strerror():
    for code in range(6):
        assert L.flce_strerror(code) and L.flce_strerror(code) != "unknown error code"
    assert L.flce_strerror(99) == "unknown error code"


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_plan_invariants(name):
    c = synth.CONFIGS[name]
    dt = L.FLCE_DTYPE_BF16 if c.dtype == "bf16" else L.FLCE_DTYPE_F32
    es = 2 if c.dtype == "bf16" else 4
    p = L.flce_plan(c.N, c.H, c.V, dt)
    half = (c.N + 1) // 2
    assert p.chunk_rows <= half and p.n_chunks >= 2
    assert p.chunk_rows % 256 == 0 or p.chunk_rows == half
    assert p.n_chunks == -(-c.N // p.chunk_rows)
    assert p.vocab_padded % 256 == 0 and p.vocab_padded - 256 < c.V <= p.vocab_padded
    assert p.logits_chunk_bytes == p.chunk_rows * p.vocab_padded * es
    # the transient never reaches the size of the full [N, V] logits
    assert p.logits_chunk_bytes < c.N * c.V * es
    assert p.grad_W_bytes == 4 * c.V * c.H
    assert L.flce_workspace_size(c.N, c.H, c.V, dt) == p.workspace_bytes
    # planning again with exactly that many bytes reproduces the plan
    q = L.flce_plan(c.N, c.H, c.V, dt, p.workspace_bytes)
    assert q.as_dict() == p.as_dict()


def _split_stats(C, H, Vp, es, s):
    tiles = -(-C // 256) * -(-H // 256)
    ksteps = Vp * es // 128
    per = -(-ksteps // s)
    real = -(-ksteps // per)
    waves = -(-(tiles * real) // 256)
    return tiles * real / (waves * 256), waves, ksteps // real


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_plan_grad_h_split(name):
    """The grad_h split has the best wave efficiency over the 256 CUs among
    splits of >= 64 K steps; among equally efficient ones it is the smallest
    with >= 12 waves of tiles >= 256 K steps long when one exists, else the
    smallest."""
    c = synth.CONFIGS[name]
    dt = L.FLCE_DTYPE_BF16 if c.dtype == "bf16" else L.FLCE_DTYPE_F32
    es = 2 if c.dtype == "bf16" else 4
    p = L.flce_plan(c.N, c.H, c.V, dt)
    ksteps = p.vocab_padded * es // 128
    cands = [s for s in range(1, 17) if s == 1 or ksteps // s >= 64]
    stats = {s: _split_stats(p.chunk_rows, c.H, p.vocab_padded, es, s) for s in cands}
    best = max(e for e, _, _ in stats.values())
    eff, waves, steps = _split_stats(p.chunk_rows, c.H, p.vocab_padded, es, p.split_k)
    assert eff >= best - 1e-9
    long_enough = [s for s in cands if stats[s][0] >= best - 1e-9 and stats[s][1] >= 12 and stats[s][2] >= 256]
    if long_enough:
        assert waves >= 12 and steps >= 256
    # the splits the page shapes get
    assert p.split_k == {"c1": 1, "c2": 2, "c3": 4, "c4": 8, "c5": 2}[name]


def test_default_budget_leaves_room_for_the_packed_rows():
    """The packed copy of h is as large as h; the default budget bounds the chunk
    transients and adds the packed rows on top, so a long batch still plans."""
    N, H, V = 1 << 20, 8192, 128256
    p = L.flce_plan(N, H, V, L.FLCE_DTYPE_BF16)
    assert p.n_chunks >= 2 and p.chunk_rows <= (N + 1) // 2
    packed = N * (H * 2 + 20)
    assert packed < p.workspace_bytes <= (16 << 30) + packed + (1 << 20)
    assert L.flce_fwd_workspace_size(N, H, V, L.FLCE_DTYPE_BF16) > packed


def test_plan_budget_shrinks_chunks():
    c = synth.CONFIGS["c4"]
    full = L.flce_plan(c.N, c.H, c.V, 0)
    small = L.flce_plan(c.N, c.H, c.V, 0, full.workspace_bytes // 3)
    assert small.chunk_rows < full.chunk_rows and small.workspace_bytes <= full.workspace_bytes // 3
    with pytest.raises(L.FlceError) as e:
        L.flce_plan(c.N, c.H, c.V, 0, 1 << 16)
    assert e.value.code == L.FLCE_EWORKSPACE


def test_plan_small_and_degenerate():
    p = L.flce_plan(1, 8, 5, 0)
    assert (p.chunk_rows, p.n_chunks) == (1, 1)
    p = L.flce_plan(0, 8, 5, 0)
    assert (p.chunk_rows, p.n_chunks) == (0, 0)
    p = L.flce_plan(600, 320, 1000, 0)
    assert (p.chunk_rows, p.n_chunks) == (256, 3)
    p = L.flce_plan(300, 64, 100, 1)
    assert (p.chunk_rows, p.n_chunks) == (150, 2)


def test_plan_rejects():
    for args, code in [((-1, 8, 8, 0), L.FLCE_EINVAL), ((4, 0, 8, 0), L.FLCE_EINVAL),
                       ((4, 8, 0, 0), L.FLCE_EINVAL), ((4, 8, 8, 7), L.FLCE_EINVAL),
                       ((4, 12, 8, 0), L.FLCE_EUNSUPPORTED), ((4, 6, 8, 1), L.FLCE_EUNSUPPORTED),
                       # 256-row tiles are addressed with 32-bit byte offsets
                       ((4, 2 ** 21 + 8, 8, 0), L.FLCE_EUNSUPPORTED),
                       ((4, 8, 2 ** 22 - 255, 0), L.FLCE_EUNSUPPORTED),
                       ((4, 8, 2 ** 21 - 255, 1), L.FLCE_EUNSUPPORTED)]:
        with pytest.raises(L.FlceError) as e:
            L.flce_plan(*args)
        assert e.value.code == code, args
        assert L.flce_workspace_size(*args) == 0


def test_plan_accepts_the_largest_shapes():
    for args in [(4, 2 ** 21, 8, 0), (4, 8, 2 ** 22 - 256, 0), (4, 8, 2 ** 21 - 256, 1)]:
        p = L.flce_plan(*args, budget_bytes=1 << 40)
        assert p.vocab_padded >= args[2]


def test_accumulator_sizes_match_the_pages():
    """The fp32 [vocab, hidden] accumulator the plan reports equals the sizes
    the pages print (tests/golden/pages_sizes.json)."""
    fx = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_sizes.json")))
    for a in fx["accumulators"]:
        p = L.flce_plan(4096, a["hidden"], a["vocab"], 0)
        b = p.grad_W_bytes if a["dtype"] == "fp32" else p.grad_W_bytes // 2
        if a.get("unit") == "GiB":
            b = b / 2**30
        assert a["bytes_lo"] <= b <= a["bytes_hi"], a


def _call(**kw):
    args = dict(h=16, W=16, labels=8, N=4, H=8, V=8, ignore_index=-100, softcap_T=0.0,
                multiplier=1.0, reduction=0, loss=4, grad_h=16, grad_W=16, n_correct=None,
                stream=0, dtype=0, workspace=256, workspace_bytes=64)
    args.update(kw)
    return L.flce_fwd_bwd(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), L.FLCE_EINVAL),
    (dict(reduction=2), L.FLCE_EINVAL),   # none needs flce_fwd_bwd_ex with loss_rows
    (dict(reduction=3), L.FLCE_EINVAL),
    (dict(N=-1), L.FLCE_EINVAL),
    (dict(H=0), L.FLCE_EINVAL),
    (dict(V=0), L.FLCE_EINVAL),
    (dict(W=None), L.FLCE_EINVAL),
    (dict(grad_W=None), L.FLCE_EINVAL),
    (dict(loss=None), L.FLCE_EINVAL),
    (dict(workspace=None), L.FLCE_EINVAL),
    (dict(h=None), L.FLCE_EINVAL),
    (dict(labels=None), L.FLCE_EINVAL),
    (dict(grad_h=None), L.FLCE_EINVAL),
    (dict(h=24), L.FLCE_EINVAL),          # misaligned
    (dict(W=8), L.FLCE_EINVAL),
    (dict(workspace=512 + 16), L.FLCE_EINVAL),
    (dict(labels=12), L.FLCE_EINVAL),
    (dict(softcap_T=float("nan")), L.FLCE_EINVAL),
    (dict(softcap_T=float("inf")), L.FLCE_EINVAL),
    (dict(multiplier=float("inf")), L.FLCE_EINVAL),
    (dict(softcap_T=1e-39), L.FLCE_EINVAL),               # 1 / T overflows
    (dict(softcap_T=1e-30, multiplier=1e10), L.FLCE_EINVAL),   # m / T overflows
    (dict(H=12), L.FLCE_EUNSUPPORTED),
    (dict(), L.FLCE_EWORKSPACE),
])
def test_fwd_bwd_rejects_before_launch(kw, code):
    # Every pointer here is a fake address.  The base arguments already fail
    # the workspace check (64 bytes), so no variant can reach a launch; each
    # variant must be rejected by its own, earlier check.
    assert _call(**kw) == code


def _opts(**kw):
    o = L.flce_options_t()
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def _call_ex(opts, **kw):
    args = dict(h=16, W=16, labels=8, N=4, H=8, V=8, ignore_index=-100, softcap_T=0.0,
                multiplier=1.0, reduction=0, loss=4, grad_h=16, grad_W=16, n_correct=None,
                stream=0, dtype=0, workspace=256, workspace_bytes=64)
    args.update(kw)
    return L.flce_fwd_bwd_ex(*args.values(), opts)


@pytest.mark.parametrize("opts,kw,code", [
    (None, dict(reduction=2), L.FLCE_EINVAL),                       # none without loss_rows
    (_opts(lse_rows=64), dict(reduction=2), L.FLCE_EINVAL),
    (_opts(loss_rows=64, grad_rows=64), dict(reduction=0), L.FLCE_EINVAL),   # row grads need none
    (_opts(loss_rows=66), dict(reduction=2), L.FLCE_EINVAL),         # misaligned
    (_opts(pred_rows=68), {}, L.FLCE_EINVAL),
    (_opts(loss_rows=64, grad_rows=66), dict(reduction=2), L.FLCE_EINVAL),
    (_opts(grad_scale=float("nan"), use_grad_scale=1), {}, L.FLCE_EINVAL),
    (_opts(grad_scale=float("inf"), use_grad_scale=1), {}, L.FLCE_EINVAL),
    (_opts(use_grad_scale=2), {}, L.FLCE_EINVAL),
    (_opts(accumulate_grad_W=2), {}, L.FLCE_EINVAL),
    (None, dict(grad_W=None), L.FLCE_EINVAL),
    (None, {}, L.FLCE_EWORKSPACE),
    # a scale that is not in use is not looked at
    (_opts(grad_scale=float("nan")), {}, L.FLCE_EWORKSPACE),
    (_opts(grad_scale=0.0, use_grad_scale=1), {}, L.FLCE_EWORKSPACE),
    (_opts(loss_rows=64, lse_rows=64, pred_rows=64, grad_rows=64, grad_scale=2.0, accumulate_grad_W=1,
           use_grad_scale=1), dict(reduction=2), L.FLCE_EWORKSPACE),
])
def test_fwd_bwd_ex_rejects_before_launch(opts, kw, code):
    # fake addresses and a 64-byte workspace: nothing can reach a launch
    assert _call_ex(opts, **kw) == code


def _call_fwd(opts, **kw):
    args = dict(h=16, W=16, labels=8, N=4, H=8, V=8, ignore_index=-100, softcap_T=0.0,
                multiplier=1.0, reduction=0, loss=4, n_correct=None, stream=0, dtype=0,
                workspace=256, workspace_bytes=64)
    args.update(kw)
    return L.flce_fwd(*args.values(), opts)


@pytest.mark.parametrize("opts,kw,code", [
    (None, dict(reduction=2), L.FLCE_EINVAL),
    (None, dict(W=None), L.FLCE_EINVAL),
    (None, dict(loss=None), L.FLCE_EINVAL),
    (None, dict(h=24), L.FLCE_EINVAL),
    (_opts(lse_rows=66), {}, L.FLCE_EINVAL),
    (None, dict(H=12), L.FLCE_EUNSUPPORTED),
    (None, {}, L.FLCE_EWORKSPACE),
    # gradient-only options are ignored by the forward-only entry
    (_opts(loss_rows=64, grad_rows=66, grad_scale=float("nan"), accumulate_grad_W=7), dict(reduction=2),
     L.FLCE_EWORKSPACE),
])
def test_fwd_rejects_before_launch(opts, kw, code):
    assert _call_fwd(opts, **kw) == code


def test_forward_only_plan_is_smaller_and_unchunked():
    for N, H, V, dt in [(8192, 6656, 202048, 0), (32768, 7168, 129280, 0), (256, 128, 1024, 1), (1, 8, 8, 0)]:
        fb = L.flce_workspace_size(N, H, V, dt)
        fo = L.flce_fwd_workspace_size(N, H, V, dt)
        assert 0 < fo < fb
        # one chunk of all N rows: header + 4 row arrays + 3 partial arrays of [V/256, N],
        # plus the packed valid rows: position, row, label, row gradient and the h copy
        nvt = (V + 255) // 256
        es = 2 if dt == 0 else 4
        assert fo >= 256 + 4 * 4 * N + 3 * 4 * nvt * N + (4 + 4 + 8 + 4) * N + N * H * es
        # the full call holds the same packed rows on top of its logits transient
        assert fb >= fo + ((N + 1) // 2) * nvt * 256 * es - 3 * 4 * nvt * N
    # no logits transient: the c4 forward workspace is the 109 MB packed copy of h
    # plus 78 MB of row arrays and partials, under 0.2 GB
    assert L.flce_fwd_workspace_size(8192, 6656, 202048, 0) < 2e8
    assert L.flce_fwd_workspace_size(4, 12, 8, 0) == 0          # unsupported H


def _call_logits(**kw):
    # base: H = 12 is unsupported for bf16 and is checked last, so no variant
    # (all with fake addresses) can reach a launch
    args = dict(h=16, W=16, N=4, H=12, V=8, softcap_T=0.0, multiplier=1.0, logits=256, ld_logits=8,
                stream=0, dtype=0)
    args.update(kw)
    return L.flce_logits(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), L.FLCE_EINVAL),
    (dict(N=-1), L.FLCE_EINVAL),
    (dict(V=0), L.FLCE_EINVAL),
    (dict(W=None), L.FLCE_EINVAL),
    (dict(W=8), L.FLCE_EINVAL),
    (dict(h=None), L.FLCE_EINVAL),
    (dict(logits=None), L.FLCE_EINVAL),
    (dict(logits=264), L.FLCE_EINVAL),          # misaligned
    (dict(ld_logits=7), L.FLCE_EINVAL),         # ld < V
    (dict(ld_logits=12), L.FLCE_EINVAL),        # 24-byte rows
    (dict(softcap_T=float("nan")), L.FLCE_EINVAL),
    (dict(), L.FLCE_EUNSUPPORTED),
])
def test_logits_rejects_before_launch(kw, code):
    assert _call_logits(**kw) == code


def _call_ce(opts=None, **kw):
    args = dict(logits=256, ld_logits=8, labels=8, N=4, V=8, ignore_index=-100, reduction=0, loss=4,
                n_correct=None, grad_logits=None, ld_grad=8, stream=0, dtype=0, workspace=256,
                workspace_bytes=64)
    args.update(kw)
    return L.flce_cross_entropy(*args.values(), opts)


@pytest.mark.parametrize("opts,kw,code", [
    (None, dict(dtype=2), L.FLCE_EINVAL),
    (None, dict(reduction=3), L.FLCE_EINVAL),
    (None, dict(reduction=2), L.FLCE_EINVAL),          # none without loss_rows
    (None, dict(N=-1), L.FLCE_EINVAL),
    (None, dict(loss=None), L.FLCE_EINVAL),
    (None, dict(workspace=None), L.FLCE_EINVAL),
    (None, dict(logits=None), L.FLCE_EINVAL),
    (None, dict(labels=12), L.FLCE_EINVAL),
    (None, dict(ld_logits=4), L.FLCE_EINVAL),
    (None, dict(grad_logits=512, ld_grad=12), L.FLCE_EINVAL),
    (None, dict(grad_logits=256, ld_grad=16, ld_logits=8), L.FLCE_EINVAL),   # in place needs equal ld
    (_opts(grad_rows=64), {}, L.FLCE_EINVAL),
    (_opts(grad_scale=float("inf"), use_grad_scale=1), {}, L.FLCE_EINVAL),
    (_opts(use_grad_scale=3), {}, L.FLCE_EINVAL),
    (None, {}, L.FLCE_EWORKSPACE),
    (_opts(grad_scale=float("inf")), {}, L.FLCE_EWORKSPACE),   # not in use: not looked at
    (_opts(loss_rows=64, grad_rows=64), dict(reduction=2, grad_logits=256), L.FLCE_EWORKSPACE),
])
def test_cross_entropy_rejects_before_launch(opts, kw, code):
    assert _call_ce(opts, **kw) == code


def test_cross_entropy_workspace_size():
    assert L.flce_cross_entropy_workspace_size(0) == 256
    assert L.flce_cross_entropy_workspace_size(1) == 256 + 3 * 256
    assert L.flce_cross_entropy_workspace_size(8192) == 256 + 3 * 8192 * 4
    assert L.flce_cross_entropy_workspace_size(-1) == 0


def test_read_status_null():
    assert L.flce_read_status(None, 0) == L.FLCE_EINVAL


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the package before torch must not map a second HIP runtime
    (torch's bundled one plus the system one): pointers and streams of one
    runtime are invalid in the other.  Runs on the CPU: only the libraries
    mapped into a fresh process are inspected."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import linear_cross_entropy_gemm_amd\nimport torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    maps = eval(out.stdout.strip().splitlines()[-1])
    assert len(maps) == 1, maps


def _call_scale(**kw):
    args = dict(grad_scale=4, grad_h_in=16, grad_h_out=16, n_h=8, h_dtype=0, grad_W_in=1 << 20,
                grad_W_out=2 << 20, n_W=8, w_dtype=0, stream=0)
    args.update(kw)
    return L.flce_scale_grads(*args.values())


@pytest.mark.parametrize("kw", [
    dict(grad_scale=None), dict(grad_scale=6),                 # null / misaligned scale
    dict(n_h=-1), dict(n_W=-1), dict(h_dtype=2), dict(w_dtype=5),
    dict(grad_h_in=None), dict(grad_h_out=24), dict(grad_W_in=None), dict(grad_W_out=(2 << 20) + 8),
    dict(grad_h_out=32, n_h=16),                                  # partly overlaps grad_h_in (16 bytes in)
    dict(grad_W_out=(1 << 20) + 16),                              # bf16 out inside the fp32 input
    dict(grad_W_out=1 << 20),                                     # bf16 out over its own fp32 input
    dict(grad_W_out=(1 << 20) + 16, w_dtype=1),                   # fp32: only exactly in place
])
def test_scale_grads_rejects_before_launch(kw):
    """flce_scale_grads checks its pointers, sizes, dtypes and overlaps on the
    host.  The addresses are fake and the call has no workspace to fail on, so
    a check that let one through would launch: CPU hosts only."""
    from conftest import gpu_available
    if gpu_available():
        pytest.skip("fake device addresses: run on a host without a GPU")
    assert _call_scale(**kw) == L.FLCE_EINVAL


def test_plan_budget_shrinks_the_split_before_the_chunk():
    """Under a budget that binds, the planner first gives up grad_h splits
    (their fp32 partials) and only then chunk rows."""
    N, H, V = 4096, 4096, 128256
    assert L.flce_plan(N, H, V, 0).split_k == 2
    a = L.flce_plan(N, H, V, 0, 300 << 20)
    assert (a.chunk_rows, a.split_k) == (768, 6) and a.workspace_bytes <= 300 << 20
    b = L.flce_plan(N, H, V, 0, a.workspace_bytes - 1)
    assert b.chunk_rows == a.chunk_rows and b.split_k < a.split_k
    assert b.workspace_bytes <= a.workspace_bytes - 1


def test_n_valid_offset_matches_the_header():
    text = open(os.path.join(ROOT, "include", "flce.h")).read()
    m = re.search(r"#define\s+FLCE_WS_N_VALID_OFFSET\s+(\d+)", text)
    assert m and int(m.group(1)) == L.WS_N_VALID_OFFSET


def test_n_valid_view_reads_the_workspace_bytes():
    """The token-accuracy denominator is a view of the workspace bytes the
    device writes (no copy): on a host tensor, the view reads what sits at
    FLCE_WS_N_VALID_OFFSET, and token_accuracy divides by it (0 / 0 -> 0)."""
    import torch
    from linear_cross_entropy_gemm_amd import torch_api
    ws = torch.zeros(256, dtype=torch.uint8)
    o = L.WS_N_VALID_OFFSET
    ws[o:o + 8] = torch.tensor([7782], dtype=torch.int64).view(torch.uint8)
    nv = torch_api._n_valid_view(ws)
    assert nv.dim() == 0 and int(nv) == 7782
    ws[o:o + 8] = torch.tensor([41], dtype=torch.int64).view(torch.uint8)
    assert int(nv) == 41   # a view: the next call's value shows through

    class R:
        n_correct = torch.tensor(10, dtype=torch.int64)
        n_valid = nv
    assert float(L.token_accuracy(R)) == 10 / 41
    ws[o:o + 8] = 0
    R.n_correct = torch.tensor(0, dtype=torch.int64)
    assert float(L.token_accuracy(R)) == 0.0
