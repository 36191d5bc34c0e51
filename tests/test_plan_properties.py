"""Property checks of the chunk planner over random shapes and budgets (host
only, no launch).  The plan keeps the token-chunk transients instead of the
[tokens, vocab] logits (DeepSeek-V3 page, Memory), so whatever the shape or
budget, a plan it returns must describe chunks that tile the batch, stay below
the whole batch, fit the budget, and be reproducible from its own workspace
size."""
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

L = pytest.importorskip("linear_cross_entropy_gemm_amd")

TILE = 256


def _shape():
    # H keeps 16-byte rows (8 bf16 or 4 fp32 values per chunk of a row)
    return st.tuples(st.integers(0, 1 << 17), st.integers(1, 2048), st.integers(1, 1 << 18),
                     st.sampled_from([L.FLCE_DTYPE_BF16, L.FLCE_DTYPE_F32])).map(
        lambda t: (t[0], t[1] * (8 if t[3] == L.FLCE_DTYPE_BF16 else 4), t[2], t[3]))


def _plan(N, H, V, dt, budget):
    try:
        return L.flce_plan(N, H, V, dt, budget) if budget is not None else L.flce_plan(N, H, V, dt)
    except L.FlceError as e:
        # a shape the kernels support only fails for lack of workspace
        assert e.code == L.FLCE_EWORKSPACE and budget is not None, (N, H, V, dt, budget, e.code)
        return None


@settings(max_examples=400, deadline=None, derandomize=True, database=None)
@given(shape=_shape(), budget=st.one_of(st.none(), st.integers(1 << 16, 1 << 36)))
def test_plan_properties(shape, budget):
    N, H, V, dt = shape
    p = _plan(N, H, V, dt, budget)
    if p is None:
        return
    es = 2 if dt == L.FLCE_DTYPE_BF16 else 4
    if N == 0:
        assert (p.chunk_rows, p.n_chunks) == (0, 0)
        return
    half = (N + 1) // 2
    assert 1 <= p.chunk_rows <= max(1, half)
    if N >= 2:
        assert p.n_chunks >= 2 and p.chunk_rows < N   # the whole batch's logits never exist
    # whole row tiles, unless the chunk is the half batch or the budget forced it below a tile
    assert p.chunk_rows % TILE == 0 or p.chunk_rows == half or p.chunk_rows < TILE
    assert p.n_chunks == -(-N // p.chunk_rows)
    assert p.vocab_padded % TILE == 0 and V <= p.vocab_padded < V + TILE
    assert p.logits_chunk_bytes == p.chunk_rows * p.vocab_padded * es
    assert p.grad_W_bytes == 4 * V * H
    assert p.split_k >= 1
    if budget is not None:
        assert p.workspace_bytes <= budget
    else:
        assert L.flce_workspace_size(N, H, V, dt) == p.workspace_bytes
    # planning again with exactly the workspace the plan needs reproduces it
    assert L.flce_plan(N, H, V, dt, p.workspace_bytes).as_dict() == p.as_dict()


@settings(max_examples=150, deadline=None, derandomize=True, database=None)
@given(shape=_shape(), b1=st.integers(1 << 20, 1 << 34), b2=st.integers(1 << 20, 1 << 34))
def test_a_larger_budget_never_gives_smaller_chunks(shape, b1, b2):
    N, H, V, dt = shape
    lo, hi = min(b1, b2), max(b1, b2)
    p_lo, p_hi = _plan(N, H, V, dt, lo), _plan(N, H, V, dt, hi)
    if p_lo is None:
        return
    assert p_hi is not None
    assert p_hi.chunk_rows >= p_lo.chunk_rows
