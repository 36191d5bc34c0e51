"""flce_fwd_bwd_noalloc, the entry point for callers that cannot allocate
device memory (static 256 MiB scratch instead of a workspace argument),
against flce_fwd_bwd_ex on the same inputs, through the C ABI.

* Two calls in a row, the second on a smaller input (the scratch keeps the
  first call's contents): loss within 2e-3 (bf16) / 1e-5 (fp32) relative,
  grad_h and grad_W within 2e-2 / 1e-4 relative Frobenius, n_correct equal;
  bitwise equal where both entry points plan the same chunks.
* A c2-sized call (N=4096, H=4096, V=128256) whose workspace plan would not
  fit the scratch: the noalloc call plans smaller chunks and still matches.
* The status output: FLCE_OK, and FLCE_ELABEL after a label outside [0, V).
* Host checks (no GPU): arguments are rejected before anything is enqueued,
  and sizes whose smallest plan exceeds the scratch return FLCE_ESCRATCH.
"""
import pytest

import synth
from gpu_util import log, rel_fro, to_device, tolerances

L = pytest.importorskip("linear_cross_entropy_gemm_amd")
IGN = synth.IGNORE_INDEX


def _raw_noalloc(**kw):
    args = dict(h=16, W=16, labels=8, N=4, H=8, V=8, ignore_index=IGN, softcap_T=0.0, multiplier=1.0,
                reduction=0, loss=4, grad_h=16, grad_W=16, n_correct=None, status=None, stream=0, dtype=0,
                options=None)
    args.update(kw)
    return L.flce_fwd_bwd_noalloc(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), L.FLCE_EINVAL),
    (dict(reduction=2), L.FLCE_EINVAL),
    (dict(W=None), L.FLCE_EINVAL),
    (dict(h=24), L.FLCE_EINVAL),
    (dict(status=6), L.FLCE_EINVAL),                       # misaligned status word
    (dict(softcap_T=float("nan")), L.FLCE_EINVAL),
    (dict(H=12), L.FLCE_EUNSUPPORTED),
    # packed rows alone (32768 x 8192 bf16 = 512 MiB) exceed the 256 MiB scratch
    (dict(N=32768, H=8192, V=1000), L.FLCE_ESCRATCH),
    # fp32: the packed rows (16384 x 4096 x 4 bytes) fill the scratch alone
    (dict(N=16384, H=4096, V=8, dtype=1), L.FLCE_ESCRATCH),
])
def test_noalloc_rejects_before_launch(kw, code):
    """Fake device addresses: every case must fail on the host, so this runs
    only where no GPU is visible (a check that let one through would
    launch)."""
    from conftest import gpu_available
    if gpu_available():
        pytest.skip("fake device addresses: run on a host without a GPU")
    assert _raw_noalloc(**kw) == code
    assert L.flce_strerror(L.FLCE_ESCRATCH) != "unknown error code"
    assert L.NOALLOC_SCRATCH_BYTES == 256 << 20


def _workspace_call(h, W, lab, N, H, V, T, m, red, dtype):
    import torch
    o = L.fwd_bwd(h, W, lab, IGN, T if T > 0 else None, m, red)
    torch.cuda.synchronize()
    return o


def _noalloc_call(h, W, lab, N, H, V, T, m, red, dtype):
    import torch
    dev = h.device
    loss = torch.empty((), dtype=torch.float32, device=dev)
    gh = torch.empty((N, H), dtype=h.dtype, device=dev)
    gW = torch.empty((V, H), dtype=torch.float32, device=dev)
    nc = torch.empty((), dtype=torch.int64, device=dev)
    st = torch.full((1,), -1, dtype=torch.int32, device=dev)
    red_code = {"mean": L.FLCE_REDUCTION_MEAN, "sum": L.FLCE_REDUCTION_SUM}[red]
    rc = L.flce_fwd_bwd_noalloc(h.data_ptr(), W.data_ptr(), lab.data_ptr(), N, H, V, IGN, float(T), float(m),
                                red_code, loss.data_ptr(), gh.data_ptr(), gW.data_ptr(), nc.data_ptr(),
                                st.data_ptr(), torch.cuda.current_stream().cuda_stream, dtype, None)
    torch.cuda.synchronize()
    assert rc == L.FLCE_OK, L.flce_strerror(rc)
    return loss, gh, gW, nc, int(st.item())


def _compare(tag, case, ref, got, N, H, V, dtype):
    loss, gh, gW, nc, st = got
    lt, gt = tolerances(case.cfg.dtype)
    e_loss = abs(loss.item() - ref.loss.item()) / max(abs(ref.loss.item()), 1e-30)
    e_gh = rel_fro(gh.float().cpu().numpy(), ref.grad_h.float().cpu().numpy())
    e_gW = rel_fro(gW.cpu().numpy(), ref.grad_W.cpu().numpy())
    plan_ws = L.flce_plan(N, H, V, dtype)
    plan_na = L.flce_plan(N, H, V, dtype, L.NOALLOC_SCRATCH_BYTES)
    same_plan = (plan_ws.chunk_rows, plan_ws.split_k) == (plan_na.chunk_rows, plan_na.split_k)
    import torch
    bitwise = (torch.equal(gh, ref.grad_h.reshape(N, H)) and torch.equal(gW, ref.grad_W)
               and loss.item() == ref.loss.item())
    log(f"[noalloc] {tag}: N={N} H={H} V={V} chunks {plan_na.chunk_rows}x{plan_na.n_chunks} split "
        f"{plan_na.split_k} (workspace plan {plan_ws.chunk_rows}x{plan_ws.n_chunks} split {plan_ws.split_k}): "
        f"loss rel {e_loss:.2e}, grad_h {e_gh:.2e}, grad_W {e_gW:.2e}, n_correct {nc.item()} vs "
        f"{ref.n_correct.item()}, status {st}, bitwise {bitwise}")
    assert st == L.FLCE_OK
    assert e_loss <= lt and e_gh <= gt and e_gW <= gt
    assert nc.item() == ref.n_correct.item()
    if same_plan:
        assert bitwise


def _case(base, N, H, V, T, m, red):
    kw = dict(softcap_T=T, multiplier=m, reduction=red)
    if synth.CONFIGS[base].seq_len:
        kw["seq_len"] = max(1, N // 4)
    return synth.make_case(synth.small_config(base, **kw), N=N, H=H, V=V)


@pytest.mark.gpu
@pytest.mark.usefixtures("require_gpu")
def test_noalloc_matches_the_workspace_entry_point():
    """Two calls in a row on one GPU, the second smaller, then a call whose
    plan is bounded by the scratch, then an fp32 call."""
    calls = [
        ("first", _case("c4", 1000, 448, 2100, 30.0, 0.5, "mean")),
        ("second, smaller", _case("c2", 300, 256, 777, 1.0, 0.37, "sum")),
        ("c2-sized, chunks bounded by the scratch", synth.make_case(synth.CONFIGS["c2"])),
        ("fp32", _case("c1", 257, 64, 530, 2.0, 1.0, "mean")),
    ]
    for tag, case in calls:
        c = case.cfg
        N, H, V = case.h.shape[0], case.h.shape[1], case.W.shape[0]
        dtype = L.FLCE_DTYPE_BF16 if c.dtype == "bf16" else L.FLCE_DTYPE_F32
        h, W, lab = to_device(case)
        got = _noalloc_call(h, W, lab, N, H, V, c.softcap_T, c.multiplier, c.reduction, dtype)
        ref = _workspace_call(h, W, lab, N, H, V, c.softcap_T, c.multiplier, c.reduction, dtype)
        _compare(tag, case, ref, got, N, H, V, dtype)


@pytest.mark.gpu
@pytest.mark.usefixtures("require_gpu")
def test_noalloc_reports_bad_labels_in_its_status_word():
    import torch
    case = _case("c2", 300, 256, 777, 1.0, 0.37, "mean")
    h, W, lab = to_device(case)
    bad = lab.clone()
    bad[17] = 777
    got = _noalloc_call(h, W, bad, 300, 256, 777, 1.0, 0.37, "mean", L.FLCE_DTYPE_BF16)
    assert got[4] == L.FLCE_ELABEL
    got = _noalloc_call(h, W, lab, 300, 256, 777, 1.0, 0.37, "mean", L.FLCE_DTYPE_BF16)
    assert got[4] == L.FLCE_OK
    torch.cuda.synchronize()


@pytest.mark.gpu
@pytest.mark.usefixtures("require_gpu")
def test_noalloc_call_replays_from_a_captured_graph():
    """The use the entry point is for: a call captured into a HIP graph (it
    allocates nothing and records only kernels), replayed several times with
    the program's own work and synchronisations in between; every replay
    equals the eager call bitwise, and the inputs changed in place between
    replays are picked up."""
    import torch
    case = _case("c4", 700, 256, 1100, 30.0, 0.5, "mean")
    c = case.cfg
    N, H, V = 700, 256, 1100
    h, W, lab = to_device(case)
    dev = h.device
    loss = torch.empty((), dtype=torch.float32, device=dev)
    gh = torch.empty((N, H), dtype=h.dtype, device=dev)
    gW = torch.empty((V, H), dtype=torch.float32, device=dev)
    nc = torch.empty((), dtype=torch.int64, device=dev)
    st = torch.full((1,), -1, dtype=torch.int32, device=dev)

    def call():
        rc = L.flce_fwd_bwd_noalloc(h.data_ptr(), W.data_ptr(), lab.data_ptr(), N, H, V, IGN, c.softcap_T,
                                    c.multiplier, L.FLCE_REDUCTION_MEAN, loss.data_ptr(), gh.data_ptr(),
                                    gW.data_ptr(), nc.data_ptr(), st.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream, L.FLCE_DTYPE_BF16, None)
        assert rc == L.FLCE_OK

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        call()                      # eager: also looks up the scratch on this device
    torch.cuda.synchronize()
    eager = (loss.clone(), gh.clone(), gW.clone(), nc.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    h0 = h.clone()
    for rep in range(4):
        loss.zero_(); gh.zero_(); gW.zero_(); nc.zero_(); st.fill_(-1)
        if rep == 3:
            h.mul_(-1.0)            # new inputs in the captured buffers
        graph.replay()
        torch.cuda.synchronize()
        if rep < 3:
            want = eager
        else:
            call()                  # eager on the new inputs, for comparison
            torch.cuda.synchronize()
            want = (loss.clone(), gh.clone(), gW.clone(), nc.clone())
            loss.zero_(); gh.zero_(); gW.zero_(); nc.zero_()
            graph.replay()
            torch.cuda.synchronize()
        got = (loss, gh, gW, nc)
        same = [torch.equal(x, y) for x, y in zip(got, want)]
        log(f"[noalloc] graph replay {rep}: bitwise equal {same}, status {int(st.item())}")
        assert all(same) and int(st.item()) == L.FLCE_OK
        # the program's own work between replays
        o = L.fwd_bwd(h, W, lab, IGN, c.softcap_T, c.multiplier, "mean")
        torch.cuda.synchronize()
        assert o.loss.item() == want[0].item()
    h.copy_(h0)
