"""The main entry point under HIP graph capture.  With a caller-owned
workspace and outputs, ``flce_fwd_bwd_ex`` allocates nothing, synchronises
nothing and records only kernels (no memset nodes), so a training step can
capture it once and replay it: every replay must equal the eager call
bitwise, with the program's own work and synchronisations between replays,
and inputs changed in place between replays must be picked up."""
import pytest

import synth
from gpu_util import log, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]

IGN = synth.IGNORE_INDEX


@pytest.mark.parametrize("rows", [False, True], ids=["packed", "row_outputs"])
def test_fwd_bwd_replays_from_a_captured_graph(rows):
    import torch
    import linear_cross_entropy_gemm_amd as L
    cfg = synth.small_config("c4", softcap_T=30.0, multiplier=0.5, reduction="mean")
    case = synth.make_case(cfg, N=700, H=256, V=1100, seed=21)
    h, W, lab = to_device(case)
    ws = torch.empty(L.flce_workspace_size(700, 256, 1100, L.FLCE_DTYPE_BF16), dtype=torch.uint8, device=h.device)

    def call(out=None):
        return L.fwd_bwd(h, W, lab, IGN, 30.0, 0.5, "mean", workspace=ws, out=out, check=False,
                         row_outputs=rows)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o = call()                  # eager, allocating the outputs the graph reuses
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    names = ["loss", "grad_h", "grad_W", "n_correct"] + (["loss_rows", "lse_rows", "pred_rows"] if rows else [])
    eager = {k: getattr(o, k).clone() for k in names}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o)
    torch.cuda.synchronize()
    h0 = h.clone()
    for rep in range(4):
        for k in names:
            getattr(o, k).zero_()
        if rep == 3:
            h.mul_(-1.0)            # new inputs in the captured buffers
            fresh = L.fwd_bwd(h, W, lab, IGN, 30.0, 0.5, "mean", row_outputs=rows)
            torch.cuda.synchronize()
            want = {k: getattr(fresh, k).clone() for k in names}
        else:
            want = eager
        graph.replay()
        torch.cuda.synchronize()
        same = {k: torch.equal(getattr(o, k), want[k]) for k in names}
        log(f"[graph] replay {rep} (row outputs {rows}): bitwise equal {same}")
        assert all(same.values())
        L.read_status(ws)           # the status word of the replay: no bad label
        # the program's own work between replays
        x = L.forward(h, W, lab, IGN, 30.0, 0.5, "mean")
        torch.cuda.synchronize()
        assert x.loss.item() == want["loss"].item()
    h.copy_(h0)
