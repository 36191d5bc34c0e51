// Chunk planner: chooses the token chunk C and lays out the workspace.
//
// The chunk's logits [C, Vp] are the largest transient ("chunked transients"
// in place of the [tokens, vocab] logits, Liger-Kernel DeepSeek-V3 page,
// Memory).  C is the largest multiple of the 256-row tile with
// C <= ceil(N / 2) whose workspace fits the budget, so every call with N >= 2
// runs at least two chunks and the full logits never exist.  With 288 GB of
// HBM per MI355X the default budget (16 GiB for the transients, plus the packed
// rows below) never binds for the lm_head shapes of the pages (Muse Glimmer
// 6656 x 202048, DeepSeek-V3 7168 x 129280).
//
// The forward-only plan stores no logits at all (only 12 bytes of partials
// per token and 256-vocabulary tile), so its chunk is as large as the budget
// allows, up to all N rows.
//
// Both plans also hold a packed copy of the valid (non-ignored) rows of h
// with their labels: ignored rows add nothing to the loss or the gradients,
// so the GEMMs can run over the valid rows alone, chunked in packed order.
#include <algorithm>

#include "flce_internal.hpp"

namespace flce {

namespace {

constexpr size_t kDefaultBudget = size_t(16) << 30;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// grad_h = G W has K = vocabulary, long and narrow output: the split rule
// (grad_h_split) applied to a full chunk of C rows, up to 16 splits.
int64_t choose_split(int64_t C, int64_t H, int64_t Vp, int64_t es) {
  const int64_t tiles = ((C + kRowTile - 1) / kRowTile) * ((H + 255) / 256);
  return grad_h_split(tiles, Vp * es / 128, 16).splits;
}

void layout(Plan* p) {
  size_t off = kHeaderBytes;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t N = size_t(p->N);
  p->off_lse = take(N * 4);
  p->off_zlab = take(N * 4);
  p->off_loss_row = take(N * 4);
  p->off_pred = take(N * 4);
  const size_t part = size_t(p->nvt) * size_t(p->C) * 4;
  p->off_pmax = take(part);
  p->off_psum = take(part);
  p->off_parg = take(part);
  if (p->fwd_only) {
    p->off_z = p->off_ghpart = 0;
  } else {
    p->off_z = take(size_t(p->C) * size_t(p->Vp) * size_t(p->es));
    // grad_h partials in whole 256 x 256 fp32 tiles (accumulator order)
    const size_t tiles = size_t((p->C + kRowTile - 1) / kRowTile) * size_t((p->H + 255) / 256);
    p->off_ghpart = take(size_t(p->split_k) * tiles * 65536 * 4);
  }
  // valid-row packing (used unless every row's log-sum-exp or argmax is
  // requested): the GEMMs then run over the non-ignored rows only
  p->off_pcnt = take(size_t((p->N + kPackRows - 1) / kPackRows) * 4);
  p->off_ppos = take(N * 4);
  p->off_prow = take(N * 4);
  p->off_plab = take(N * 8);
  p->off_pgrow = take(N * 4);
  p->off_ph = take(N * size_t(p->H) * size_t(p->es));
  p->total = off;
}

}  // namespace

int make_plan(int64_t N, int64_t H, int64_t V, int dtype, size_t budget, bool fwd_only, Plan* out) {
  if (!out) return FLCE_EINVAL;
  if (dtype != FLCE_DTYPE_BF16 && dtype != FLCE_DTYPE_F32) return FLCE_EINVAL;
  if (N < 0 || H < 1 || V < 1) return FLCE_EINVAL;
  const int64_t es = dtype == FLCE_DTYPE_BF16 ? 2 : 4;
  if ((H * es) % 16 != 0) return FLCE_EUNSUPPORTED;
  // The GEMM loaders address a 256-row tile of an operand or of grad_W
  // (fp32) with 32-bit byte offsets: 256 rows of H or Vp elements must stay
  // within 2^31 bytes.
  const int64_t lim_h = (int64_t(1) << 31) / (int64_t(kRowTile) * 4);
  const int64_t lim_v = (int64_t(1) << 31) / (int64_t(kRowTile) * es) - kVocabTile;
  if (N > (int64_t(1) << 31) - 1 || H > lim_h || V > lim_v) return FLCE_EUNSUPPORTED;
  // The default budget bounds the chunk transients; the packed copy of the
  // valid rows (as large as h itself) and its row arrays come on top of it.
  if (budget == 0)
    budget = kDefaultBudget + size_t(N) * (size_t(H) * size_t(es) + 20) +
             size_t((N + kPackRows - 1) / kPackRows) * 4 + size_t(256) * 8;

  Plan p{};
  p.N = N;
  p.H = H;
  p.V = V;
  p.es = es;
  p.Vp = (V + kVocabTile - 1) / kVocabTile * kVocabTile;
  p.nvt = p.Vp / kVocabTile;
  p.fwd_only = fwd_only;
  if (N == 0) {
    p.C = 0;
    p.n_chunks = 0;
    p.split_k = 1;
    layout(&p);
    if (p.total > budget) return FLCE_EWORKSPACE;
    *out = p;
    return FLCE_OK;
  }
  const int64_t top = fwd_only ? N : (N + 1) / 2;
  const int64_t ksteps = p.Vp * es / 128;
  // The planner's chunk and grad_h split, or, when the budget binds, fewer
  // splits (smaller fp32 partials) before a smaller chunk.
  auto fits = [&](int64_t c) {
    p.C = c;
    p.n_chunks = (N + c - 1) / c;
    const int64_t pick = choose_split(c, H, p.Vp, es);
    for (int64_t s = pick; s >= 1; --s) {
      const int64_t per = (ksteps + s - 1) / s;
      const int64_t real = (ksteps + per - 1) / per;
      if (s < pick && real == p.split_k) continue;   // same split as the last one tried
      p.split_k = real;
      layout(&p);
      if (p.total <= budget) return true;
      if (fwd_only) break;   // no partials: the split does not change the size
    }
    return false;
  };
  // Whether some split fits depends on c alone (with one split the
  // workspace grows with c), so the largest fitting chunk is found by
  // bisection: multiples of the row tile first, then halving below one tile.
  int64_t c = top < kRowTile ? top : top / kRowTile * kRowTile;
  if (fits(c)) {
    *out = p;
    return FLCE_OK;
  }
  if (c > kRowTile) {
    int64_t lo = 0, hi = c / kRowTile;   // tiles: hi does not fit; lo fits (0: none known)
    while (hi - lo > 1) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (fits(mid * kRowTile))
        lo = mid;
      else
        hi = mid;
    }
    if (lo > 0 && fits(lo * kRowTile)) {
      *out = p;
      return FLCE_OK;
    }
  }
  for (c = std::min<int64_t>(c, kRowTile) / 2; c >= 1; c /= 2) {
    if (fits(c)) {
      *out = p;
      return FLCE_OK;
    }
  }
  return FLCE_EWORKSPACE;
}

}  // namespace flce
