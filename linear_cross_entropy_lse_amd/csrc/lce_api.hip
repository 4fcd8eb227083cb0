// C-ABI entry points of liblce (declared in include/lce.h): argument checks,
// workspace layout and the launch sequence of the forward and backward passes.
// No device memory is ever allocated here; everything lives in the caller's
// workspace.
#include <algorithm>
#include <cstdlib>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/lce.h"
#include "lce_device.h"
#include "lce_internal.h"

namespace lce {
namespace {

// Plans are computed for the 256 compute units of the gfx950 MI355X, so the
// workspace size depends on the shape only.
constexpr int kTargetCUs = 256;
constexpr size_t kAlign = 256;
// The fused variant keeps a Nc x V logits block; its 256-row tiles use 32-bit
// offsets (256·V·2 bytes < 2^31).
constexpr int64_t kFusedMaxV = (int64_t)1 << 21;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool options_ok(const lce_options* o) {
  if (!o) return false;
  const bool finite = std::isfinite(o->softcap) && std::isfinite(o->logit_scale) &&
                      std::isfinite(o->label_smoothing) && std::isfinite(o->z_loss) &&
                      std::isfinite(o->filter_eps);
  return finite && o->logit_scale > 0.0f && o->label_smoothing >= 0.0f &&
         o->label_smoothing <= 1.0f && o->z_loss >= 0.0f && o->reduction >= LCE_REDUCE_MEAN &&
         o->reduction <= LCE_REDUCE_NONE && o->filter_eps >= 0.0f &&
         (o->precise == 0 || o->precise == 1);
}

bool shape_ok(int64_t N, int64_t H, int64_t V) {
  return N >= 0 && N < INT_MAX && H >= 8 && H < (1 << 20) && H % 8 == 0 && V >= 1 && V < INT_MAX;
}

// Vocabulary splits of a persistent (token tile, split) grid of T token
// tiles: as many as fit T·S <= kTargetCUs, so the grid is one wave of
// workgroups.  The forward calls it with at most kGroupTiles token tiles per
// launch; the logit-gradient grid past kGroupTiles uses rounds instead
// (grad_round_splits).
int pick_splits(int T, int n_vtiles) {
  int S = kTargetCUs / std::max(T, 1);
  S = std::max(1, std::min(S, n_vtiles));
  return S;
}

// XCD sub-grid of a T x S (token tile, split) persistent grid: each of the 8
// XCDs takes a tt x ss block (tt | T, ss | S, (T/tt)·(S/ss) = 8), as square as
// possible, fewer token tiles on ties.  tt = 0 keeps the plain order.
void pick_xcd_grid(int T, int S, int& tt, int& ss) {
  tt = 0;
  ss = 0;
  const int nwg = T * S;
  if (nwg % 8 != 0) return;
  const int per = nwg / 8;
  int best = INT_MAX;
  for (int s = 1; s <= per; ++s) {
    if (per % s != 0 || S % s != 0) continue;
    const int t = per / s;
    if (T % t != 0 || (T / t) * (S / s) != 8) continue;
    const int score = 2 * std::abs(t - s) + (t > s ? 1 : 0);
    if (score < best) {
      best = score;
      tt = t;
      ss = s;
    }
  }
}

struct FwdPlan {
  int T, S, n_vtiles, nb_fin;
  int S_tail;          // splits of the tail launch; 0: no tail
  int64_t rows_main;   // rows of the groups split S ways (all rows without a tail)
  size_t off_state, off_target, off_pm, off_ps, off_pz, off_blocks, total;
};

// Forward: the token tiles go in groups of at most kGroupTiles (one launch
// each), every group split S ways over the vocabulary, so that a full group
// fills the 256 workgroups of the grid with a 4 x 8 block of (token tiles,
// splits) on each XCD: per pipeline step an XCD touches 4 X blocks and 8 W
// blocks.  One launch over every token tile would leave fewer splits as N
// grows (S = 256 / T) and, past 32 token tiles, blocks of 8 x 4, 16 x 2 or
// 32 x 1 tiles that share fewer operands in L2.  Past kGroupTiles tiles, the
// r = T mod kGroupTiles tiles after the last full group form a tail launch
// split pick_splits(r) ways: with the groups' S it would take as long as a
// full group for as few as one token tile.
constexpr int kGroupTiles = kTargetCUs / 8;

FwdPlan plan_forward(int64_t N, int64_t H, int64_t V) {
  (void)H;
  FwdPlan p{};
  p.T = (int)std::max<int64_t>(1, ceil_div(N, kTile));
  p.n_vtiles = (int)ceil_div(V, kTile);
  p.S = pick_splits(std::min(p.T, kGroupTiles), p.n_vtiles);
  const int tail_tiles = p.T > kGroupTiles ? p.T % kGroupTiles : 0;
  p.rows_main = tail_tiles ? (int64_t)(p.T - tail_tiles) * kTile : N;
  p.S_tail = tail_tiles ? pick_splits(tail_tiles, p.n_vtiles) : 0;
  p.nb_fin = lse_finalize_blocks(std::max<int64_t>(N, 1));
  // Split partials: [S, rows_main] for the groups, then [S_tail, N - rows_main].
  const size_t n_part = (size_t)p.rows_main * p.S + (size_t)(N - p.rows_main) * p.S_tail;
  size_t o = 0;
  p.off_state = o;   o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_target = o;  o = align_up(o + sizeof(float) * (size_t)N);
  p.off_pm = o;      o = align_up(o + sizeof(float) * n_part);
  p.off_ps = o;      o = align_up(o + sizeof(float) * n_part);
  p.off_pz = o;      o = align_up(o + sizeof(float) * n_part);
  p.off_blocks = o;  o = align_up(o + sizeof(BlockStats) * (size_t)p.nb_fin);
  p.total = std::max<size_t>(o, kAlign);
  return p;
}

struct BwdPlan {
  int T, nchunks, n_vtiles_chunk, S_chunk, nt_h, nb_prep, ksplit;
  int64_t Vc, ldg;
  size_t off_state, off_key, off_deriv, off_gs, off_c1, off_oh, off_keys_a, off_keys_b, off_head,
      off_tail, off_blocks, off_scalars, off_flags, off_G, off_dXp, off_dWs, off_Wp, off_pos1,
      off_pkey, off_labd, off_labo, off_domcol, off_domc, off_dombase, off_de, off_dkey,
      off_dkeys_a, off_dkeys_b, off_dcounts, total;
};

// Logit-gradient grid past kGroupTiles token tiles: full rounds of 256 / S
// token tiles x S splits, S in {8, 4, 2, 1} (round_tile), then the tiles left
// over in a launch of their own split pick_splits ways (a last round partly
// filled would take as long as a full one).  S is chosen for the least
// estimated time: rounds x tiles per split (the slowest workgroup of a round),
// times the measured cost of the XCD block a round gives each XCD (4 x 8 tiles
// 1, 8 x 4 1.02, 16 x 2 1.055, 32 x 1 1.25: smaller blocks share fewer
// operands in L2), plus the left-over launch's tiles per split.  Only S with
// at least one full round are considered; with none (fewer vocabulary tiles
// than 8 and fewer token tiles than a round of fewer splits) the result is 0
// and the grid is a single launch of T x pick_splits(T) workgroups.  Narrow
// chunks (large N) have few vocabulary tiles, so the splits that fill a round
// evenly can matter more than the block.
int grad_round_splits(int T, int n_vt) {
  static const int kS[4] = {8, 4, 2, 1};
  static const double kBlockCost[4] = {1.0, 1.02, 1.055, 1.25};
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < 4; ++i) {
    const int S = kS[i];
    const int rt = kTargetCUs / S;
    if (S > n_vt || T < rt) continue;
    const int rest = T % rt;
    double cost = (double)(T / rt) * ceil_div(n_vt, S) * kBlockCost[i];
    if (rest > 0) cost += (double)ceil_div(n_vt, pick_splits(rest, n_vt));
    if (cost < best_cost) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

// K parts of the dX tiles of a chunk of `steps` 64-deep K steps.  The dX
// tiles (T token tiles x nt_h hidden tiles) contract over the whole chunk, the
// dW tiles over the rows; both kinds together hold 2·T·nt_h·steps tile-steps.
// With few token tiles the dX tiles are too few and too long to spread over
// the workgroups (at N = 1024 one of them would take three times the average
// work of a workgroup), so their K range is split until one part costs no
// more than the average; part k accumulates into its own fp32 buffer and the
// parts are summed in order at the end.  Every part holds at least one step:
// the count is ceil(steps / ceil(steps / k)), which the chunk GEMM's own part
// length ceil(steps / ksplit) reproduces.
int dx_parts(int64_t steps, int T, int nt_h) {
  const int64_t avg = std::max<int64_t>(1, 2 * (int64_t)T * nt_h * steps / kTargetCUs);
  const int64_t ks = std::min<int64_t>(std::max<int64_t>(1, ceil_div(steps, avg)), 16);
  return (int)ceil_div(steps, ceil_div(steps, ks));
}

// Chunk width: the bf16 gradient chunk N x Vc is kept about as large as W
// (N·Vc ≤ V·H before its width is rounded up to whole 256-column tiles, so
// that tiles never straddle two chunks), with a floor (below) and a cap of
// 2^21 columns (a 256-row block of a chunk then spans < 2^31 bytes, the
// 32-bit buffer offsets of the gradient kernels).  The number of chunks is
// the fewest that meets the bound: ceil(N/H) between the floor and the cap,
// counted before the rounding (rounding the bound down first can add a chunk
// for a few columns: 5 chunks instead of 4 at N = 4H).
// Floor: a dW tile of the chunk GEMM contracts over all N rows (N/64 steps),
// and the chunk's work per workgroup is 2·T·nt_h·(Vc/64)/256 steps; a dW tile
// is no longer than that average when Vc ≥ 32768/nt_h columns.  Narrower
// chunks leave a few workgroups holding one dW tile each to set the time (at
// H = 1024, N = 16384: twice the average).  So the floor is 32768/nt_h
// columns in whole tiles, at least 4096 and at most 16384 (where H ≤ 512, the
// chunk then holds N·16384 bf16 values at most).  `precise`: the chunk
// holds two bf16 parts (hi, lo), twice as many chunks of half the width (the
// workspace queries return the larger of the two plans).  With a vocabulary
// order (`sorted`) the chunk's W rows are gathered into position order (Wp),
// its dW rows go through the fp32 chunk buffer, and the label keys are moved
// to positions (pos1, pkey).
BwdPlan plan_backward(int64_t N, int64_t H, int64_t V, lce_dtype dW_dtype, bool sorted = false,
                      bool precise = false) {
  BwdPlan p{};
  const int64_t Nc = std::max<int64_t>(N, 1);
  p.T = (int)ceil_div(Nc, kTile);
  const int64_t nt_h = ceil_div(H, kTile);
  const int64_t floor_cols = std::max<int64_t>(
      4096, std::min<int64_t>(16384, ceil_div(ceil_div(32768, nt_h), kTile) * kTile));
  const int64_t parts = precise ? 2 : 1, cap_cols = (int64_t)1 << 21;
  int64_t n;
  if (V * H < floor_cols * Nc)
    n = ceil_div(V * parts, floor_cols);
  else if (V * H > cap_cols * Nc)
    n = ceil_div(V * parts, cap_cols);
  else
    n = ceil_div(Nc * parts, H);
  n = std::max<int64_t>(n, 1);
  p.Vc = ceil_div(ceil_div(V, n), kTile) * kTile;
  p.nchunks = (int)ceil_div(V, p.Vc);
  p.ldg = p.Vc;
  p.n_vtiles_chunk = (int)(p.Vc / kTile);
  p.S_chunk = pick_splits(p.T, p.n_vtiles_chunk);
  p.nt_h = (int)ceil_div(H, kTile);
  p.nb_prep = row_prep_blocks(Nc);
  p.ksplit = dx_parts(ceil_div(std::min<int64_t>(p.Vc, V), kBK), p.T, p.nt_h);
  size_t o = 0;
  p.off_state = o;   o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_key = o;     o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_deriv = o;   o = align_up(o + sizeof(float) * (size_t)N);
  p.off_gs = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_c1 = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_oh = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_keys_a = o;  o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_keys_b = o;  o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_head = o;    o = align_up(o + sizeof(float) * (size_t)seg_chunks(N) * (size_t)H);
  p.off_tail = o;    o = align_up(o + sizeof(float) * (size_t)seg_chunks(N) * (size_t)H);
  p.off_blocks = o;  o = align_up(o + sizeof(BlockStats) * (size_t)p.nb_prep);
  p.off_scalars = o; o = align_up(o + 16);
  // Exact entries of the logit-gradient pass and the sort of the dominant ones.
  p.off_labd = o;    o = align_up(o + sizeof(float) * (size_t)N);
  p.off_labo = o;    o = align_up(o + sizeof(float) * (size_t)N);
  p.off_domcol = o;  o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_domc = o;    o = align_up(o + sizeof(float) * (size_t)N);
  p.off_dombase = o; o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_de = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_dkey = o;    o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_dkeys_a = o; o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_dkeys_b = o; o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_dcounts = o; o = align_up(o + 16);
  p.off_flags = o;   o = align_up(o + sizeof(uint32_t) * (size_t)p.T * (size_t)p.n_vtiles_chunk);
  // Blocked gradient chunk: T token tiles (padded) x Vc columns; with
  // `precise` its lo part follows at G + T·256·ldg.
  p.off_G = o;       o = align_up(o + sizeof(uint16_t) * (size_t)p.T * kTile * (size_t)p.ldg *
                                      (precise ? 2 : 1));
  p.off_dXp = o;     o = align_up(o + sizeof(float) * (size_t)p.ksplit * (size_t)N * (size_t)H);
  p.off_dWs = o;
  if (dW_dtype == LCE_BF16 || sorted) o = align_up(o + sizeof(float) * (size_t)p.Vc * (size_t)H);
  if (sorted) {
    p.off_Wp = o;    o = align_up(o + sizeof(uint16_t) * (size_t)p.Vc * (size_t)H);
    p.off_pos1 = o;  o = align_up(o + sizeof(int32_t) * (size_t)V);
    p.off_pkey = o;  o = align_up(o + sizeof(int32_t) * (size_t)N);
  }
  p.total = std::max<size_t>(o, kAlign);
  return p;
}

// Vocabulary order: per-block column sums of X, x̄, the key and its sort
// word per entry, and the two buffers of the merge sort.
struct OrderPlan {
  int64_t nrb;
  size_t off_part, off_cnt, off_xbar, off_key, off_word, off_keys_a, off_keys_b, total;
};

OrderPlan plan_order(int64_t N, int64_t H, int64_t V) {
  OrderPlan p{};
  p.nrb = mean_row_blocks(N);
  size_t o = 0;
  p.off_part = o;    o = align_up(o + sizeof(float) * (size_t)p.nrb * (size_t)H);
  p.off_cnt = o;     o = align_up(o + sizeof(int32_t) * (size_t)p.nrb);
  p.off_xbar = o;    o = align_up(o + sizeof(float) * (size_t)H);
  p.off_key = o;     o = align_up(o + sizeof(float) * (size_t)V);
  p.off_word = o;    o = align_up(o + sizeof(uint32_t) * (size_t)V);
  p.off_keys_a = o;  o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(V));
  p.off_keys_b = o;  o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(V));
  p.total = std::max<size_t>(o, kAlign);
  return p;
}

// Fused row-chunk variant.  Chunk rows: whole 256-row tiles, T of them in
// every chunk but the last (fused_chunk_tiles sets T and with it the chunk
// count).  The dX tiles of one chunk contract over the whole vocabulary;
// their K range is split so that one part costs no more than the average
// work per workgroup (the dW tiles contract over the chunk's rows only),
// each chunk by its own token tiles: ksplit is a full chunk's, dxp_rows
// covers the last chunk's parts too.
struct FusedPlan {
  int64_t Nc, ldu;
  int nchunks, T, S, n_vtiles, nt_h, ksplit, nb_prep, nb_fin;
  int64_t dxp_rows;   // rows x K parts of the largest chunk's dX partials
  size_t off_state, off_key, off_target, off_deriv, off_gs, off_c1, off_oh, off_rrow, off_keys_a,
      off_keys_b, off_head, off_tail, off_bprep, off_bfin, off_scalars, off_pm, off_ps, off_pz,
      off_pcz, off_pcb, off_labd, off_labo, off_domcol, off_domc, off_de, off_dkey, off_dkeys_a,
      off_dkeys_b, off_dcounts, off_U, off_ref, off_Xs, off_dXp, off_dWacc, total;
};

// Token tiles per row chunk of the fused call (every chunk but the last has
// this many).  A chunk has at most 2H rows (its bf16 logits block at most
// twice the size of W) and, from two tiles of rows on, at most half of the
// row tiles rounded up (the call never holds every row's logits at once).
// Among the fewest chunks that meet the bound and up to three more, each
// count with chunks as even as whole tiles allow, the one with the least
// estimated time is taken: the logits pass of a chunk takes ceil(n_vt / S)
// tile products on its slowest workgroup (S = pick_splits of the chunk's
// tiles), and every chunk after the first reads and rewrites the fp32 dW once
// more, about V / 16384 tile products (8·V·H bytes at the bandwidth against
// 2·256²·H flops at one compute unit's MFMA rate, both about 5·10^12 per
// second).  The chunk GEMM's work does not depend on the chunking.  Even
// chunks keep a short last chunk from costing a whole dW pass for a few rows.
int fused_chunk_tiles(int64_t N, int64_t H, int64_t V) {
  const int64_t T_all = ceil_div(std::max<int64_t>(N, 1), kTile);
  const int n_vt = (int)ceil_div(V, kTile);
  const int64_t half = T_all >= 2 ? ceil_div(T_all, 2) : 1;
  const int64_t lim = std::max<int64_t>(1, std::min<int64_t>(2 * H / kTile, half));
  const int64_t n_min = ceil_div(T_all, lim);
  const double dw_pass = (double)V / 16384.0;
  int64_t best = ceil_div(T_all, n_min);
  double best_cost = 1e300;
  for (int64_t n = n_min; n <= n_min + 3 && n <= T_all; ++n) {
    const int64_t t = ceil_div(T_all, n), last = T_all - (n - 1) * t;
    if (last <= 0) continue;
    const double cost = (double)(n - 1) * ceil_div(n_vt, pick_splits((int)t, n_vt)) +
                        (double)ceil_div(n_vt, pick_splits((int)last, n_vt)) + (double)(n - 1) * dw_pass;
    if (cost < best_cost) {
      best_cost = cost;
      best = t;
    }
  }
  return (int)best;
}

FusedPlan plan_fused(int64_t N, int64_t H, int64_t V, lce_dtype dW_dtype) {
  FusedPlan p{};
  const int64_t Np = ceil_div(std::max<int64_t>(N, 1), kTile) * kTile;
  p.T = fused_chunk_tiles(N, H, V);
  p.Nc = (int64_t)p.T * kTile;
  p.nchunks = (int)ceil_div(std::max<int64_t>(N, 1), p.Nc);
  p.n_vtiles = (int)ceil_div(V, kTile);
  p.ldu = (int64_t)p.n_vtiles * kTile;
  p.S = pick_splits(p.T, p.n_vtiles);
  p.nt_h = (int)ceil_div(H, kTile);
  // K parts of each chunk's dX tiles (dx_parts of the chunk's own token
  // tiles: a short last chunk has few dX tiles, each over the whole
  // vocabulary, and takes more parts), at a part stride of the chunk's rows.
  const int64_t steps = ceil_div(V, kBK);
  const int64_t last_rows = std::max<int64_t>(N, 1) - (int64_t)(p.nchunks - 1) * p.Nc;
  p.ksplit = dx_parts(steps, p.T, p.nt_h);
  p.dxp_rows = std::max<int64_t>(p.ksplit * p.Nc,
                                 dx_parts(steps, (int)ceil_div(last_rows, kTile), p.nt_h) * last_rows);
  p.nb_prep = row_prep_blocks(std::max<int64_t>(N, 1));
  p.nb_fin = lse_finalize_blocks(Np);
  size_t o = 0;
  p.off_state = o;   o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_key = o;     o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_target = o;  o = align_up(o + sizeof(float) * (size_t)N);
  p.off_deriv = o;   o = align_up(o + sizeof(float) * (size_t)N);
  p.off_gs = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_c1 = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_oh = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_rrow = o;    o = align_up(o + sizeof(float) * (size_t)N);
  p.off_keys_a = o;  o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_keys_b = o;  o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_head = o;    o = align_up(o + sizeof(float) * (size_t)seg_chunks(N) * (size_t)H);
  p.off_tail = o;    o = align_up(o + sizeof(float) * (size_t)seg_chunks(N) * (size_t)H);
  p.off_bprep = o;   o = align_up(o + sizeof(BlockStats) * (size_t)p.nb_prep);
  p.off_bfin = o;    o = align_up(o + sizeof(BlockStats) * (size_t)p.nb_fin);
  p.off_scalars = o; o = align_up(o + 16);
  // Split partials: a shorter last chunk takes more splits (S·rows stays
  // below kTargetCUs·256).
  const size_t part = (size_t)kTargetCUs * kTile;
  p.off_pm = o;      o = align_up(o + sizeof(float) * part);
  p.off_ps = o;      o = align_up(o + sizeof(float) * part);
  p.off_pz = o;      o = align_up(o + sizeof(float) * part);
  // Dominant-entry candidates per split, and the exact entries (as the
  // recompute path's).
  p.off_pcz = o;     o = align_up(o + sizeof(float) * part);
  p.off_pcb = o;     o = align_up(o + sizeof(int32_t) * part);
  p.off_labd = o;    o = align_up(o + sizeof(float) * (size_t)N);
  p.off_labo = o;    o = align_up(o + sizeof(float) * (size_t)N);
  p.off_domcol = o;  o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_domc = o;    o = align_up(o + sizeof(float) * (size_t)N);
  p.off_de = o;      o = align_up(o + sizeof(float) * (size_t)N);
  p.off_dkey = o;    o = align_up(o + sizeof(int32_t) * (size_t)N);
  p.off_dkeys_a = o; o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_dkeys_b = o; o = align_up(o + sizeof(uint64_t) * (size_t)sort_padded(N));
  p.off_dcounts = o; o = align_up(o + 16);
  p.off_U = o;       o = align_up(o + sizeof(uint16_t) * (size_t)p.Nc * (size_t)p.ldu);
  p.off_ref = o;     o = align_up(o + sizeof(float) * (size_t)p.Nc * 2 * (size_t)p.n_vtiles);
  p.off_Xs = o;      o = align_up(o + sizeof(uint16_t) * (size_t)p.Nc * (size_t)H);
  p.off_dXp = o;     o = align_up(o + sizeof(float) * (size_t)p.dxp_rows * (size_t)H);
  p.off_dWacc = o;
  if (dW_dtype == LCE_BF16) o = align_up(o + sizeof(float) * (size_t)V * (size_t)H);
  p.total = std::max<size_t>(o, kAlign);
  return p;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// ---------------------------------------------------------------------------
// Optional kernel timing: hipEvent pairs around each launch on its stream.
// ---------------------------------------------------------------------------
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<std::string> names;
  std::vector<int64_t> launches;
  std::vector<double> total_ms;
  struct Pending { int id; hipEvent_t a, b; };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;

  int id_of(const char* name) {
    for (size_t i = 0; i < names.size(); ++i)
      if (names[i] == name) return (int)i;
    names.emplace_back(name);
    launches.push_back(0);
    total_ms.push_back(0.0);
    return (int)names.size() - 1;
  }
  hipError_t take(hipEvent_t* e) {
    if (!pool.empty()) {
      *e = pool.back();
      pool.pop_back();
      return hipSuccess;
    }
    return hipEventCreate(e);
  }
};

Timing& timing() {
  static Timing t;
  return t;
}

// Runs `launch` (which enqueues one kernel on `stream`), bracketed by events
// when timing is enabled.
template <class F>
hipError_t timed(const char* name, hipStream_t stream, F&& launch) {
  Timing& t = timing();
  bool on;
  {
    std::lock_guard<std::mutex> g(t.mu);
    on = t.on;
  }
  if (!on) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> g(t.mu);
    hipError_t e = t.take(&a);
    if (e != hipSuccess) return e;
    e = t.take(&b);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipEventRecord(a, stream);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, stream);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(t.mu);
  t.pending.push_back({t.id_of(name), a, b});
  return hipSuccess;
}

#define LCE_TRY(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return LCE_ERR_HIP; \
  } while (0)

#define LCE_LAUNCH(name, stream, call) LCE_TRY(timed(name, stream, [&]() { return call; }))

// ---------------------------------------------------------------------------
// Library-held scratch of lce_forward_noalloc: one fixed array per device,
// shared by every call on that device.  Host code never passes the array's
// name to a kernel (in host code it is only a stand-in for the symbol); it
// passes the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_for_current_device(void** ptr) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *ptr = ptrs[dev];
  return hipSuccess;
}

bool range_ok(int64_t V, int64_t v_lo, int64_t V_total) {
  return v_lo >= 0 && V_total < INT_MAX && v_lo <= V_total - V;
}

LossTerms loss_terms(const lce_options* opt, int64_t V_total, const float* part_z) {
  LossTerms t{};
  t.one_minus_eps = 1.0f - opt->label_smoothing;
  t.eps_over_v = (float)((double)opt->label_smoothing / (double)V_total);
  t.z_loss = opt->z_loss;
  t.part_z = part_z;
  return t;
}

// Outputs of a forward pass.  The full forward sets loss, reduced and
// n_valid; a vocabulary shard's forward sets target (and optionally zsum)
// instead and leaves reduced null.
struct FwdOut {
  float* loss = nullptr;
  float* lse = nullptr;
  float* reduced = nullptr;
  int32_t* n_valid = nullptr;
  int32_t* bad_label = nullptr;
  float* target = nullptr;
  float* zsum = nullptr;
};

lce_status forward_impl(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                        int64_t N, int64_t H, int64_t V, VocabRange vr, const lce_options* opt,
                        const FwdOut& out, void* workspace_dev, size_t workspace_bytes,
                        void* stream_ptr) {
  if (N > 0 && (!X_dev || !W_dev || !labels_dev || !workspace_dev)) return LCE_ERR_INVALID_ARG;
  if (!aligned(X_dev, 16) || !aligned(W_dev, 16) || !aligned(labels_dev, 8) ||
      !aligned(workspace_dev, kAlign))
    return LCE_ERR_ALIGNMENT;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const bool shard = out.reduced == nullptr;
  if (N == 0) {
    if (!shard)
      LCE_LAUNCH("empty_forward", stream, launch_empty_forward(out.reduced, out.n_valid, out.bad_label, stream));
    return LCE_OK;
  }
  const FwdPlan pl = plan_forward(N, H, V);
  if (workspace_bytes < pl.total) return LCE_ERR_WORKSPACE;

  int32_t* state = at<int32_t>(workspace_dev, pl.off_state);
  float* target = out.target ? out.target : at<float>(workspace_dev, pl.off_target);
  float* pm = at<float>(workspace_dev, pl.off_pm);
  float* ps = at<float>(workspace_dev, pl.off_ps);
  float* pz = at<float>(workspace_dev, pl.off_pz);
  BlockStats* blocks = at<BlockStats>(workspace_dev, pl.off_blocks);
  const uint16_t* X = static_cast<const uint16_t*>(X_dev);
  const uint16_t* W = static_cast<const uint16_t*>(W_dev);
  // Per-row logit sums: for label smoothing, or when a shard reports them.
  const bool zsum = shard ? out.zsum != nullptr : opt->label_smoothing > 0.0f;

  LCE_LAUNCH("row_prep", stream, launch_row_prep(X, W, labels_dev, N, H, V, vr, opt->ignore_index, opt->softcap,
                          opt->logit_scale, state, nullptr, target, nullptr, nullptr, stream));
  // Launches over the rows [r0, r0 + n) split S ways, partials [S, ldp] from
  // offset `part` of the partial buffers.
  auto partials = [&](int64_t r0, int64_t n, int S, size_t part, int64_t ldp) -> hipError_t {
    LseParams lp{};
    lp.X = X + r0 * H; lp.W = W; lp.N = n; lp.H = H; lp.V = V;
    lp.T = (int)ceil_div(n, kTile); lp.S = S; lp.n_vtiles = pl.n_vtiles;
    lp.softcap = opt->softcap; lp.logit_scale = opt->logit_scale;
    pick_xcd_grid(lp.T, lp.S, lp.tt, lp.ss);
    lp.part_m = pm + part; lp.part_s = ps + part; lp.part_z = zsum ? pz + part : nullptr;
    lp.ldp = ldp;
    return launch_lse_partials(lp, stream);
  };
  // Final LSE and loss of the rows [r0, r0 + n) from S partials [S, n] at
  // offset `part` (r0 is a multiple of 256, the rows of one block of sums).
  auto finalize = [&](int64_t r0, int64_t n, int S, size_t part) -> hipError_t {
    const LossTerms terms = loss_terms(opt, vr.V_total, zsum ? pz + part : nullptr);
    return launch_lse_finalize(pm + part, ps + part, S, n, state + r0, target + r0, terms,
                               out.lse + r0, out.loss ? out.loss + r0 : nullptr,
                               shard ? nullptr : blocks + r0 / kTile,
                               out.zsum ? out.zsum + r0 : nullptr, stream);
  };
  const int64_t group_rows = (int64_t)kGroupTiles * kTile, tail_rows = N - pl.rows_main;
  const size_t tail_part = (size_t)pl.rows_main * pl.S;
  for (int64_t r0 = 0; r0 < pl.rows_main; r0 += group_rows)
    LCE_LAUNCH("lse_partials", stream, partials(r0, std::min(group_rows, pl.rows_main - r0), pl.S,
                                                (size_t)r0, pl.rows_main));
  if (tail_rows > 0)
    LCE_LAUNCH("lse_partials", stream, partials(pl.rows_main, tail_rows, pl.S_tail, tail_part, tail_rows));
  LCE_LAUNCH("lse_finalize", stream, finalize(0, pl.rows_main, pl.S, 0));
  if (tail_rows > 0)
    LCE_LAUNCH("lse_finalize", stream, finalize(pl.rows_main, tail_rows, pl.S_tail, tail_part));
  if (!shard)
    LCE_LAUNCH("mean_finalize", stream, launch_mean_finalize(blocks, pl.nb_fin, opt->reduction == LCE_REDUCE_MEAN,
                                  out.reduced, out.n_valid, out.bad_label, stream));
  return LCE_OK;
}

// Backward over the vocabulary rows W holds ([vr.v_lo, vr.v_lo + V) of
// vr.V_total): their rows of dW and their share of dX.
// `order`: null, or a device permutation of [0, V) (the vocabulary order of
// the sorted backward; full vocabulary only).
lce_status backward_impl(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                         const float* lse_dev, const float* dloss_dev, int64_t N, int64_t H,
                         int64_t V, VocabRange vr, const int32_t* order, const lce_options* opt,
                         void* dX_dev, lce_dtype dX_dtype, void* dW_dev, lce_dtype dW_dtype,
                         void* workspace_dev, size_t workspace_bytes, void* stream_ptr) {
  if (!options_ok(opt)) return LCE_ERR_INVALID_ARG;
  if (opt->filter_eps > 0.0f && (opt->label_smoothing > 0.0f || opt->precise))
    return LCE_ERR_INVALID_ARG;
  if ((dX_dtype != LCE_F32 && dX_dtype != LCE_BF16) || (dW_dtype != LCE_F32 && dW_dtype != LCE_BF16))
    return LCE_ERR_INVALID_ARG;
  if (!dW_dev) return LCE_ERR_INVALID_ARG;
  if (N > 0 && (!X_dev || !W_dev || !labels_dev || !lse_dev || !dloss_dev || !dX_dev ||
                !workspace_dev))
    return LCE_ERR_INVALID_ARG;
  if (!aligned(X_dev, 16) || !aligned(W_dev, 16) || !aligned(labels_dev, 8) ||
      !aligned(lse_dev, 4) || !aligned(dloss_dev, 4) || !aligned(dX_dev, 16) ||
      !aligned(dW_dev, 16) || !aligned(workspace_dev, kAlign))
    return LCE_ERR_ALIGNMENT;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const int64_t dw_bytes = V * H * (dW_dtype == LCE_BF16 ? 2 : 4);
  if (N == 0) {
    LCE_LAUNCH("fill_zero", stream, launch_fill_zero(dW_dev, dw_bytes, stream));
    return LCE_OK;
  }
  const bool sorted = order != nullptr;
  const bool precise = opt->precise != 0;
  const BwdPlan pl = plan_backward(N, H, V, dW_dtype, sorted, precise);
  if (workspace_bytes < pl.total) return LCE_ERR_WORKSPACE;

  int32_t* state = at<int32_t>(workspace_dev, pl.off_state);
  int32_t* key = at<int32_t>(workspace_dev, pl.off_key);
  float* deriv = at<float>(workspace_dev, pl.off_deriv);
  float* gs = at<float>(workspace_dev, pl.off_gs);
  float* c1 = at<float>(workspace_dev, pl.off_c1);
  float* oh = at<float>(workspace_dev, pl.off_oh);
  uint64_t* keys_a = at<uint64_t>(workspace_dev, pl.off_keys_a);
  uint64_t* keys_b = at<uint64_t>(workspace_dev, pl.off_keys_b);
  const uint64_t* keys = sort_passes(N) % 2 == 0 ? keys_a : keys_b;   // where the sort ends
  float* part_head = at<float>(workspace_dev, pl.off_head);
  float* part_tail = at<float>(workspace_dev, pl.off_tail);
  BlockStats* blocks = at<BlockStats>(workspace_dev, pl.off_blocks);
  float* scalars = at<float>(workspace_dev, pl.off_scalars);       // [0] plain scale, [1] = 1
  int32_t* counts = at<int32_t>(workspace_dev, pl.off_scalars + 8);
  uint16_t* G = at<uint16_t>(workspace_dev, pl.off_G);
  uint16_t* G_lo = precise ? G + (size_t)pl.T * kTile * (size_t)pl.ldg : nullptr;
  uint32_t* flags = opt->filter_eps > 0.0f ? at<uint32_t>(workspace_dev, pl.off_flags) : nullptr;
  float* dXp = at<float>(workspace_dev, pl.off_dXp);
  float* dWs = at<float>(workspace_dev, pl.off_dWs);
  uint16_t* Wp = sorted ? at<uint16_t>(workspace_dev, pl.off_Wp) : nullptr;
  int32_t* pos1 = sorted ? at<int32_t>(workspace_dev, pl.off_pos1) : nullptr;
  int32_t* pkey = sorted ? at<int32_t>(workspace_dev, pl.off_pkey) : nullptr;
  const uint16_t* X = static_cast<const uint16_t*>(X_dev);
  const uint16_t* W = static_cast<const uint16_t*>(W_dev);
  // The plain path stores G = p·d and applies one scalar scale afterwards; label
  // smoothing, Z-loss or a per-row upstream gradient need the general form.
  // While every row has the same scale (no per-row upstream gradient, no
  // Z-loss), that scale stays a scalar applied in fp32 after the contractions
  // in the general form too, so the bf16 rounding of G never sees it.
  const bool general = opt->label_smoothing > 0.0f || opt->z_loss > 0.0f ||
                       opt->reduction == LCE_REDUCE_NONE;
  const bool unit = opt->reduction != LCE_REDUCE_NONE && opt->z_loss == 0.0f;
  const float* gemm_scale = unit ? scalars : scalars + 1;
  // The label's entry and a dominant entry of each row skip the bf16 chunk
  // and are applied in fp32 (launch_exact_entries): oh comes from their
  // values, and the dominant entries get a sorted dW correction of their own,
  // like the one-hot term's.
  float* lab_dense = at<float>(workspace_dev, pl.off_labd);
  float* lab_oh = at<float>(workspace_dev, pl.off_labo);
  int32_t* dom_col = at<int32_t>(workspace_dev, pl.off_domcol);
  float* dom_coef = at<float>(workspace_dev, pl.off_domc);
  int32_t* dom_base = at<int32_t>(workspace_dev, pl.off_dombase);
  float* de = at<float>(workspace_dev, pl.off_de);
  int32_t* dkey = at<int32_t>(workspace_dev, pl.off_dkey);
  uint64_t* dkeys_a = at<uint64_t>(workspace_dev, pl.off_dkeys_a);
  uint64_t* dkeys_b = at<uint64_t>(workspace_dev, pl.off_dkeys_b);
  const uint64_t* dkeys = sort_passes(N) % 2 == 0 ? dkeys_a : dkeys_b;
  int32_t* dcounts = at<int32_t>(workspace_dev, pl.off_dcounts);
  const int32_t* lab_key = sorted ? pkey : key;
  // oh, de and the sorted dominant keys from the exact entries written so far.
  auto exact_terms = [&]() -> lce_status {
    LCE_LAUNCH("exact_coef", stream, launch_exact_coef(state, lab_key, lab_dense, lab_oh, dom_col, dom_coef,
                                                      unit ? scalars : nullptr, N, oh, de, dkey, stream));
    LCE_LAUNCH("sort_dominant", stream, launch_sort_by_label(dkey, N, dkeys_a, dkeys_b, stream));
    LCE_LAUNCH("count_dominant", stream, launch_count_keys(dkeys, N, dcounts, stream));
    return LCE_OK;
  };

  LCE_LAUNCH("row_prep", stream, launch_row_prep(X, W, labels_dev, N, H, V, vr, opt->ignore_index, opt->softcap,
                          opt->logit_scale, state, key, nullptr, deriv, blocks, stream));
  LCE_LAUNCH("scale_finalize", stream, launch_scale_finalize(blocks, pl.nb_prep, dloss_dev, opt->reduction == LCE_REDUCE_MEAN,
                                opt->logit_scale, scalars, counts, stream));
  LCE_LAUNCH("row_coef", stream, launch_row_coef(state, lse_dev, deriv, opt->reduction == LCE_REDUCE_NONE ? dloss_dev : nullptr,
                          scalars, N, opt->logit_scale, 1.0f - opt->label_smoothing, opt->z_loss,
                          unit, general ? gs : nullptr, general ? c1 : nullptr, oh, lab_dense,
                          lab_oh, dom_col, dom_base, stream));
  // With an order, the one-hot correction of dW works in positions: the label
  // keys are moved to the positions of the labels before the sort.
  if (sorted)
    LCE_LAUNCH("position_keys", stream, launch_position_keys(order, V, key, N, pos1, pkey, stream));
  LCE_LAUNCH("sort_by_label", stream, launch_sort_by_label(sorted ? pkey : key, N, keys_a, keys_b, stream));
  // The label entries' values, once for the whole vocabulary (their logits
  // as the tile kernels form them, from W's own rows); each chunk then only
  // clears their slots in G.
  {
    ExactParams ep{};
    ep.X = X; ep.W = W; ep.N = N; ep.H = H; ep.V = V;
    ep.v_begin = 0; ep.chunk_len = V; ep.key_offset = 0;
    ep.softcap = opt->softcap; ep.logit_scale = opt->logit_scale;
    ep.lse = lse_dev; ep.row_state = state; ep.row_key = key;
    ep.gs = general ? gs : nullptr; ep.c1 = c1;
    ep.eps_over_v = (float)((double)opt->label_smoothing / (double)vr.V_total);
    ep.one_minus_eps = 1.0f - opt->label_smoothing;
    ep.label_pass = kLabelValues;
    ep.lab_dense = lab_dense; ep.lab_oh = lab_oh;
    LCE_LAUNCH("exact_labels", stream, launch_exact_entries(ep, stream));
  }

  // dX partial buffers, all written by the first chunk's chunk GEMM (the
  // widest chunk) and summed by dx_finalize.  Every chunk's parts are at most
  // dx_part_steps steps long, so a narrower last chunk has no more parts.
  const int dx_nparts = flags ? 1 : pl.ksplit;
  const int64_t dx_part_steps = ceil_div(ceil_div(std::min<int64_t>(pl.Vc, V), kBK), dx_nparts);
  for (int c = 0; c < pl.nchunks; ++c) {
    const int64_t v_begin = (int64_t)c * pl.Vc;
    const int64_t chunk_len = std::min<int64_t>(pl.Vc, V - v_begin);
    const int n_vt = (int)ceil_div(chunk_len, kTile);
    // The chunk's W rows: a slice of W, or (with an order) the rows of the
    // entries at positions [v_begin, v_begin + chunk_len), gathered.
    if (sorted)
      LCE_LAUNCH("gather_rows", stream, launch_gather_rows(W, V, H, order, v_begin, chunk_len, Wp, stream));
    const uint16_t* Wsrc = sorted ? Wp : W;
    const int64_t w_begin = sorted ? 0 : v_begin, w_rows = sorted ? chunk_len : V;

    GradParams gp{};
    gp.X = X; gp.W = Wsrc; gp.N = N; gp.H = H; gp.V = w_rows; gp.v_begin = w_begin;
    gp.T = pl.T; gp.S = std::min(pl.S_chunk, n_vt); gp.n_vtiles = n_vt;
    gp.softcap = opt->softcap; gp.logit_scale = opt->logit_scale;
    pick_xcd_grid(gp.T, gp.S, gp.tt, gp.ss);
    // Past kGroupTiles token tiles: full rounds here, the tiles left over in a
    // second launch (below).
    int rest_tiles = 0;
    const int round_splits = pl.T > kGroupTiles ? grad_round_splits(pl.T, n_vt) : 0;
    if (round_splits > 0) {
      gp.S = round_splits;
      gp.round_tiles = kTargetCUs / gp.S;
      rest_tiles = pl.T % gp.round_tiles;
      gp.T = pl.T - rest_tiles;
    }
    gp.lse = lse_dev; gp.row_state = state; gp.G = G; gp.ldg = pl.ldg;
    gp.gs = general ? gs : nullptr; gp.c1 = c1;
    gp.eps_over_v = (float)((double)opt->label_smoothing / (double)vr.V_total);
    gp.flags = reinterpret_cast<uint8_t*>(flags); gp.filter_eps = opt->filter_eps;
    gp.dom_base = dom_base; gp.key_offset = sorted ? v_begin : 0;
    gp.G_lo = G_lo;
    LCE_LAUNCH("grad_logits", stream, launch_grad_logits(gp, stream));
    if (rest_tiles > 0) {
      gp.t0 = gp.T; gp.T = rest_tiles; gp.round_tiles = 0;
      gp.S = pick_splits(rest_tiles, n_vt);
      pick_xcd_grid(gp.T, gp.S, gp.tt, gp.ss);
      LCE_LAUNCH("grad_logits", stream, launch_grad_logits(gp, stream));
    }
    ExactParams ep{};
    ep.X = X; ep.W = Wsrc; ep.N = N; ep.H = H; ep.V = w_rows;
    ep.v_begin = w_begin; ep.chunk_len = chunk_len; ep.key_offset = gp.key_offset;
    ep.n_vtiles = n_vt; ep.softcap = opt->softcap; ep.logit_scale = opt->logit_scale;
    ep.lse = lse_dev; ep.row_state = state; ep.row_key = lab_key;
    ep.gs = general ? gs : nullptr; ep.c1 = c1;
    ep.eps_over_v = gp.eps_over_v; ep.one_minus_eps = 1.0f - opt->label_smoothing;
    ep.dom_base = dom_base; ep.G = G; ep.G_lo = G_lo;
    ep.label_pass = kLabelSlots; ep.keys = keys; ep.n_keys = counts + 1;
    ep.lab_dense = lab_dense; ep.lab_oh = lab_oh; ep.dom_col = dom_col; ep.dom_coef = dom_coef;
    LCE_LAUNCH("exact_entries", stream, launch_exact_entries(ep, stream));
    // With the filter, exact dense values whose block is skipped are dropped.
    if (flags)
      LCE_LAUNCH("filter_exact", stream, launch_filter_exact(flags, n_vt, w_begin, state, lab_key,
                                                            gp.key_offset, N, lab_dense, dom_col,
                                                            dom_coef, stream));

    ChunkGemmParams cp{};
    cp.G = G; cp.ldg = pl.ldg; cp.Wc = Wsrc + w_begin * H; cp.wc_rows = w_rows - w_begin; cp.X = X;
    cp.N = N; cp.H = H; cp.chunk_len = chunk_len;
    cp.nt_tok = pl.T; cp.nt_h = pl.nt_h; cp.nt_v = n_vt;
    cp.accumulate = c > 0; cp.dX_acc = dXp; cp.scale = gemm_scale;
    // K parts of this chunk's dX tiles: as many parts of at most
    // dx_part_steps steps as the chunk needs (each part then holds at least
    // one step; the chunk GEMM's part length ceil(steps / ksplit) gives the
    // same count).  A narrower last chunk may use fewer parts, which then
    // accumulate into the first buffers.  The filter's form takes one part.
    cp.ksplit = flags ? 1 : (int)ceil_div(ceil_div(chunk_len, kBK), dx_part_steps);
    if (cp.ksplit > dx_nparts) return LCE_ERR_INVALID_ARG;   // cannot happen: chunk 0 is the widest
    cp.dx_part_stride = N * H; cp.dw_accumulate = 0; cp.flags = flags;
    cp.dW_dst = dW_dtype == LCE_F32 && !sorted ? static_cast<float*>(dW_dev) + v_begin * H : dWs;
    LCE_LAUNCH("chunk_gemm", stream, launch_chunk_gemm(cp, stream));
    if (precise) {
      // The lo part through the same contractions, added to both results.
      cp.G = G_lo; cp.accumulate = 1; cp.dw_accumulate = 1;
      LCE_LAUNCH("chunk_gemm", stream, launch_chunk_gemm(cp, stream));
    }
    if (sorted || dW_dtype == LCE_BF16) {
      // This chunk's dW rows are final once corrected: the exact entries of
      // its labels and dominant entries are all known now.
      const lce_status st = exact_terms();
      if (st != LCE_OK) return st;
      LCE_LAUNCH("dw_correct", stream, launch_dw_correct(keys, counts, oh, X, N, H, dWs, v_begin,
                                v_begin + chunk_len, part_head, part_tail, stream));
      LCE_LAUNCH("dw_correct", stream, launch_dw_correct(dkeys, dcounts, de, X, N, H, dWs, v_begin,
                                v_begin + chunk_len, part_head, part_tail, stream));
      if (sorted)
        LCE_LAUNCH("scatter_rows", stream, launch_scatter_rows(dWs, V, H, order, v_begin, chunk_len, dW_dev,
                                    dW_dtype == LCE_BF16, stream));
      else
        LCE_LAUNCH("cast_bf16", stream, launch_cast_bf16(dWs, static_cast<uint16_t*>(dW_dev) + v_begin * H,
                                 chunk_len * H, stream));
    }
  }
  if (dW_dtype == LCE_F32 && !sorted) {
    const lce_status st = exact_terms();
    if (st != LCE_OK) return st;
    LCE_LAUNCH("dw_correct", stream, launch_dw_correct(keys, counts, oh, X, N, H,
                              static_cast<float*>(dW_dev), 0, V, part_head, part_tail, stream));
    LCE_LAUNCH("dw_correct", stream, launch_dw_correct(dkeys, dcounts, de, X, N, H,
                              static_cast<float*>(dW_dev), 0, V, part_head, part_tail, stream));
  }
  LCE_LAUNCH("dx_finalize", stream, launch_dx_finalize(dXp, dx_nparts, N * H, N, H, V, state, key, oh, W, gemm_scale, nullptr,
                             dom_col, de, order, dX_dev, dX_dtype == LCE_BF16, stream));
  return LCE_OK;
}


}  // namespace
}  // namespace lce

using namespace lce;

extern "C" {

int lce_version(void) { return 100; }

void lce_timing_enable(int enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.on = enable != 0;
}

void lce_timing_reset(void) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (auto& p : t.pending) {
    (void)hipEventSynchronize(p.b);
    t.pool.push_back(p.a);
    t.pool.push_back(p.b);
  }
  t.pending.clear();
  for (size_t i = 0; i < t.names.size(); ++i) {
    t.launches[i] = 0;
    t.total_ms[i] = 0.0;
  }
}

int lce_timing_read(lce_kernel_timing* out, int max_entries) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  int rc = 0;
  for (auto& p : t.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess)
      rc = -1;
    t.launches[p.id] += 1;
    t.total_ms[p.id] += ms;
    t.pool.push_back(p.a);
    t.pool.push_back(p.b);
  }
  t.pending.clear();
  if (rc < 0) return rc;
  const int n = (int)t.names.size();
  if (out) {
    for (int i = 0; i < n && i < max_entries; ++i) {
      std::memset(out[i].name, 0, sizeof(out[i].name));
      std::strncpy(out[i].name, t.names[i].c_str(), sizeof(out[i].name) - 1);
      out[i].launches = t.launches[i];
      out[i].total_ms = t.total_ms[i];
    }
  }
  return n;
}

lce_status lce_device_info(int device, int32_t* cu_count, int32_t* clock_khz, char* arch,
                           int32_t arch_len) {
  if (!cu_count || !clock_khz) return LCE_ERR_INVALID_ARG;
  int dev = device;
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return LCE_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LCE_ERR_HIP;
  *cu_count = prop.multiProcessorCount;
  *clock_khz = prop.clockRate;
  if (arch && arch_len > 0) {
    std::strncpy(arch, prop.gcnArchName, (size_t)arch_len - 1);
    arch[arch_len - 1] = 0;
  }
  return LCE_OK;
}

lce_status lce_backward_plan(int64_t N, int64_t H, int64_t V, int32_t precise,
                             int64_t* chunk_columns, int32_t* n_chunks, int32_t* dx_parts) {
  if (!chunk_columns || !n_chunks || !dx_parts || (precise != 0 && precise != 1))
    return LCE_ERR_INVALID_ARG;
  if (!shape_ok(N, H, V)) return LCE_ERR_SHAPE;
  const BwdPlan pl = plan_backward(N, H, V, LCE_F32, false, precise != 0);
  *chunk_columns = pl.Vc;
  *n_chunks = pl.nchunks;
  *dx_parts = pl.ksplit;
  return LCE_OK;
}

lce_status lce_fused_plan(int64_t N, int64_t H, int64_t V, int64_t* chunk_rows, int32_t* n_chunks,
                          int32_t* dx_parts) {
  if (!chunk_rows || !n_chunks || !dx_parts) return LCE_ERR_INVALID_ARG;
  if (!shape_ok(N, H, V)) return LCE_ERR_SHAPE;
  const FusedPlan pl = plan_fused(N, H, V, LCE_F32);
  *chunk_rows = pl.Nc;
  *n_chunks = pl.nchunks;
  *dx_parts = pl.ksplit;
  return LCE_OK;
}

const char* lce_status_string(lce_status status) {
  switch (status) {
    case LCE_OK: return "ok";
    case LCE_ERR_INVALID_ARG: return "invalid argument (NULL pointer or enum out of range)";
    case LCE_ERR_SHAPE: return "shape out of range (need 0 <= N < 2^31 - 1, 8 <= H < 2^20, H % 8 == 0, 1 <= V < 2^31 - 1)";
    case LCE_ERR_ALIGNMENT: return "misaligned pointer (X/W/dX/dW 16 B, labels 8 B, workspace 256 B)";
    case LCE_ERR_WORKSPACE: return "workspace smaller than the size query returns";
    case LCE_ERR_HIP: return "HIP runtime error";
    case LCE_ERR_SCRATCH_LIMIT:
      return "shape needs more scratch than lce_forward_noalloc holds (lce_forward_noalloc_max_bytes)";
  }
  return "unknown status";
}

size_t lce_forward_noalloc_max_bytes(void) { return kScratchBytes; }

lce_status lce_forward_noalloc(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                               int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                               float softcap, float* loss_dev, float* lse_dev, float* mean_dev,
                               int32_t* n_valid_dev, int32_t* bad_label_dev, void* stream_ptr) {
  if (!shape_ok(N, H, V)) return LCE_ERR_SHAPE;
  if (!mean_dev || !n_valid_dev) return LCE_ERR_INVALID_ARG;
  if (N > 0 && (!X_dev || !W_dev || !labels_dev || !loss_dev || !lse_dev))
    return LCE_ERR_INVALID_ARG;
  if (!aligned(X_dev, 16) || !aligned(W_dev, 16) || !aligned(labels_dev, 8) ||
      !aligned(loss_dev, 4) || !aligned(lse_dev, 4) || !aligned(mean_dev, 4) ||
      !aligned(n_valid_dev, 4) || !aligned(bad_label_dev, 4))
    return LCE_ERR_ALIGNMENT;
  // The size check comes before any HIP call, so an oversized shape is
  // refused without touching a device.
  if (N > 0 && plan_forward(N, H, V).total > kScratchBytes) return LCE_ERR_SCRATCH_LIMIT;
  lce_options opt;
  lce_options_default(&opt);
  opt.ignore_index = ignore_index;
  opt.softcap = softcap;
  FwdOut out{};
  out.loss = loss_dev; out.lse = lse_dev; out.reduced = mean_dev;
  out.n_valid = n_valid_dev; out.bad_label = bad_label_dev;
  void* ws = nullptr;
  if (N > 0 && scratch_for_current_device(&ws) != hipSuccess) return LCE_ERR_HIP;
  return forward_impl(X_dev, W_dev, labels_dev, N, H, V, VocabRange{0, V}, &opt, out, ws,
                      kScratchBytes, stream_ptr);
}

size_t lce_forward_workspace_bytes(int64_t N, int64_t H, int64_t V) {
  if (!shape_ok(N, H, V)) return 0;
  return plan_forward(N, H, V).total;
}

size_t lce_backward_workspace_bytes(int64_t N, int64_t H, int64_t V, lce_dtype dW_dtype) {
  if (!shape_ok(N, H, V) || (dW_dtype != LCE_F32 && dW_dtype != LCE_BF16)) return 0;
  return std::max(plan_backward(N, H, V, dW_dtype).total,
                  plan_backward(N, H, V, dW_dtype, false, true).total);
}

void lce_options_default(lce_options* opt) {
  if (!opt) return;
  opt->ignore_index = -100;
  opt->softcap = 0.0f;
  opt->logit_scale = 1.0f;
  opt->label_smoothing = 0.0f;
  opt->z_loss = 0.0f;
  opt->reduction = LCE_REDUCE_MEAN;
  opt->filter_eps = 0.0f;
  opt->precise = 0;
}

lce_status lce_forward(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                       int64_t N, int64_t H, int64_t V, int64_t ignore_index, float softcap,
                       float* loss_dev, float* lse_dev, float* mean_dev, int32_t* n_valid_dev,
                       int32_t* bad_label_dev, void* workspace_dev, size_t workspace_bytes,
                       void* stream_ptr) {
  lce_options opt;
  lce_options_default(&opt);
  opt.ignore_index = ignore_index;
  opt.softcap = softcap;
  return lce_forward_ex(X_dev, W_dev, labels_dev, N, H, V, &opt, loss_dev, lse_dev, mean_dev,
                        n_valid_dev, bad_label_dev, workspace_dev, workspace_bytes, stream_ptr);
}

lce_status lce_forward_ex(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                          int64_t N, int64_t H, int64_t V, const lce_options* opt,
                          float* loss_dev, float* lse_dev, float* reduced_dev,
                          int32_t* n_valid_dev, int32_t* bad_label_dev, void* workspace_dev,
                          size_t workspace_bytes, void* stream_ptr) {
  if (!shape_ok(N, H, V)) return LCE_ERR_SHAPE;
  if (!options_ok(opt) || !reduced_dev || !n_valid_dev) return LCE_ERR_INVALID_ARG;
  if (N > 0 && (!loss_dev || !lse_dev)) return LCE_ERR_INVALID_ARG;
  if (!aligned(loss_dev, 4) || !aligned(lse_dev, 4) || !aligned(reduced_dev, 4) ||
      !aligned(n_valid_dev, 4) || !aligned(bad_label_dev, 4))
    return LCE_ERR_ALIGNMENT;
  FwdOut out{};
  out.loss = loss_dev; out.lse = lse_dev; out.reduced = reduced_dev;
  out.n_valid = n_valid_dev; out.bad_label = bad_label_dev;
  return forward_impl(X_dev, W_dev, labels_dev, N, H, V, VocabRange{0, V}, opt, out,
                      workspace_dev, workspace_bytes, stream_ptr);
}

lce_status lce_shard_forward(const void* X_dev, const void* W_shard_dev,
                             const int64_t* labels_dev, int64_t N, int64_t H, int64_t V_shard,
                             int64_t vocab_offset, int64_t vocab_total, const lce_options* opt,
                             float* lse_part_dev, float* target_part_dev, float* zsum_part_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream_ptr) {
  if (!shape_ok(N, H, V_shard) || !range_ok(V_shard, vocab_offset, vocab_total))
    return LCE_ERR_SHAPE;
  if (!options_ok(opt)) return LCE_ERR_INVALID_ARG;
  if (N > 0 && (!lse_part_dev || !target_part_dev)) return LCE_ERR_INVALID_ARG;
  if (!aligned(lse_part_dev, 4) || !aligned(target_part_dev, 4) || !aligned(zsum_part_dev, 4))
    return LCE_ERR_ALIGNMENT;
  if (N == 0) return LCE_OK;
  FwdOut out{};
  out.lse = lse_part_dev; out.target = target_part_dev; out.zsum = zsum_part_dev;
  return forward_impl(X_dev, W_shard_dev, labels_dev, N, H, V_shard,
                      VocabRange{vocab_offset, vocab_total}, opt, out, workspace_dev,
                      workspace_bytes, stream_ptr);
}

size_t lce_shard_merge_workspace_bytes(int64_t N) {
  if (N < 0 || N >= INT_MAX) return 0;
  return std::max<size_t>(align_up(sizeof(BlockStats) * (size_t)lse_finalize_blocks(std::max<int64_t>(N, 1))), kAlign);
}

lce_status lce_shard_merge(const float* lse_parts_dev, const float* target_parts_dev,
                           const float* zsum_parts_dev, int32_t n_shards,
                           const int64_t* labels_dev, int64_t N, int64_t vocab_total,
                           const lce_options* opt, float* loss_dev, float* lse_dev,
                           float* reduced_dev, int32_t* n_valid_dev, int32_t* bad_label_dev,
                           void* workspace_dev, size_t workspace_bytes, void* stream_ptr) {
  if (N < 0 || N >= INT_MAX || vocab_total < 1 || vocab_total >= INT_MAX) return LCE_ERR_SHAPE;
  if (!options_ok(opt) || n_shards < 1 || !reduced_dev || !n_valid_dev) return LCE_ERR_INVALID_ARG;
  if (N > 0 && (!lse_parts_dev || !target_parts_dev || !labels_dev || !loss_dev || !lse_dev ||
                !workspace_dev))
    return LCE_ERR_INVALID_ARG;
  const bool smoothing = opt->label_smoothing > 0.0f;
  if (N > 0 && smoothing && !zsum_parts_dev) return LCE_ERR_INVALID_ARG;
  if (!aligned(lse_parts_dev, 4) || !aligned(target_parts_dev, 4) || !aligned(zsum_parts_dev, 4) ||
      !aligned(labels_dev, 8) || !aligned(loss_dev, 4) || !aligned(lse_dev, 4) ||
      !aligned(reduced_dev, 4) || !aligned(n_valid_dev, 4) || !aligned(bad_label_dev, 4) ||
      !aligned(workspace_dev, kAlign))
    return LCE_ERR_ALIGNMENT;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  if (N == 0) {
    LCE_LAUNCH("empty_forward", stream, launch_empty_forward(reduced_dev, n_valid_dev, bad_label_dev, stream));
    return LCE_OK;
  }
  if (workspace_bytes < lce_shard_merge_workspace_bytes(N)) return LCE_ERR_WORKSPACE;
  BlockStats* blocks = static_cast<BlockStats*>(workspace_dev);
  const LossTerms terms = loss_terms(opt, vocab_total, nullptr);
  LCE_LAUNCH("shard_merge", stream, launch_shard_merge(lse_parts_dev, target_parts_dev, smoothing ? zsum_parts_dev : nullptr,
                               n_shards, labels_dev, N, vocab_total, opt->ignore_index, terms,
                               lse_dev, loss_dev, blocks, stream));
  LCE_LAUNCH("mean_finalize", stream, launch_mean_finalize(blocks, lse_finalize_blocks(N), opt->reduction == LCE_REDUCE_MEAN,
                                reduced_dev, n_valid_dev, bad_label_dev, stream));
  return LCE_OK;
}

lce_status lce_backward(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                        const float* lse_dev, const float* dloss_dev, int64_t N, int64_t H,
                        int64_t V, int64_t ignore_index, float softcap, void* dX_dev,
                        lce_dtype dX_dtype, void* dW_dev, lce_dtype dW_dtype,
                        void* workspace_dev, size_t workspace_bytes, void* stream_ptr) {
  lce_options opt;
  lce_options_default(&opt);
  opt.ignore_index = ignore_index;
  opt.softcap = softcap;
  return lce_backward_ex(X_dev, W_dev, labels_dev, lse_dev, dloss_dev, N, H, V, &opt, dX_dev,
                         dX_dtype, dW_dev, dW_dtype, workspace_dev, workspace_bytes, stream_ptr);
}

lce_status lce_backward_ex(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                           const float* lse_dev, const float* dloss_dev, int64_t N, int64_t H,
                           int64_t V, const lce_options* opt, void* dX_dev, lce_dtype dX_dtype,
                           void* dW_dev, lce_dtype dW_dtype, void* workspace_dev,
                           size_t workspace_bytes, void* stream_ptr) {
  if (!shape_ok(N, H, V)) return LCE_ERR_SHAPE;
  return backward_impl(X_dev, W_dev, labels_dev, lse_dev, dloss_dev, N, H, V, VocabRange{0, V},
                       nullptr, opt, dX_dev, dX_dtype, dW_dev, dW_dtype, workspace_dev,
                       workspace_bytes, stream_ptr);
}

size_t lce_backward_sorted_workspace_bytes(int64_t N, int64_t H, int64_t V, lce_dtype dW_dtype) {
  if (!shape_ok(N, H, V) || (dW_dtype != LCE_F32 && dW_dtype != LCE_BF16)) return 0;
  return std::max(plan_backward(N, H, V, dW_dtype, true).total,
                  plan_backward(N, H, V, dW_dtype, true, true).total);
}

lce_status lce_backward_sorted(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                               const float* lse_dev, const float* dloss_dev, int64_t N, int64_t H,
                               int64_t V, const lce_options* opt, const int32_t* order_dev,
                               void* dX_dev, lce_dtype dX_dtype, void* dW_dev, lce_dtype dW_dtype,
                               void* workspace_dev, size_t workspace_bytes, void* stream_ptr) {
  if (!shape_ok(N, H, V)) return LCE_ERR_SHAPE;
  if (!order_dev) return LCE_ERR_INVALID_ARG;
  if (!aligned(order_dev, 4)) return LCE_ERR_ALIGNMENT;
  return backward_impl(X_dev, W_dev, labels_dev, lse_dev, dloss_dev, N, H, V, VocabRange{0, V},
                       order_dev, opt, dX_dev, dX_dtype, dW_dev, dW_dtype, workspace_dev,
                       workspace_bytes, stream_ptr);
}

size_t lce_vocab_order_workspace_bytes(int64_t N, int64_t H, int64_t V) {
  if (!shape_ok(N, H, V)) return 0;
  return plan_order(N, H, V).total;
}

lce_status lce_vocab_order(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                           int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                           float* mean_logit_dev, int32_t* order_dev, void* workspace_dev,
                           size_t workspace_bytes, void* stream_ptr) {
  if (!shape_ok(N, H, V)) return LCE_ERR_SHAPE;
  if (!W_dev || !order_dev || !workspace_dev || (N > 0 && (!X_dev || !labels_dev)))
    return LCE_ERR_INVALID_ARG;
  if (!aligned(X_dev, 16) || !aligned(W_dev, 16) || !aligned(labels_dev, 8) ||
      !aligned(mean_logit_dev, 4) || !aligned(order_dev, 4) || !aligned(workspace_dev, kAlign))
    return LCE_ERR_ALIGNMENT;
  const OrderPlan pl = plan_order(N, H, V);
  if (workspace_bytes < pl.total) return LCE_ERR_WORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  float* part = at<float>(workspace_dev, pl.off_part);
  int32_t* cnt = at<int32_t>(workspace_dev, pl.off_cnt);
  float* xbar = at<float>(workspace_dev, pl.off_xbar);
  float* key = mean_logit_dev ? mean_logit_dev : at<float>(workspace_dev, pl.off_key);
  uint32_t* word = at<uint32_t>(workspace_dev, pl.off_word);
  uint64_t* keys_a = at<uint64_t>(workspace_dev, pl.off_keys_a);
  uint64_t* keys_b = at<uint64_t>(workspace_dev, pl.off_keys_b);
  LCE_LAUNCH("vocab_key", stream, launch_vocab_key(static_cast<const uint16_t*>(X_dev), labels_dev, N, H,
                                           static_cast<const uint16_t*>(W_dev), V, ignore_index,
                                           part, cnt, xbar, key, word, stream));
  LCE_LAUNCH("vocab_sort", stream, launch_sort_by_label(reinterpret_cast<const int32_t*>(word), V, keys_a,
                                                keys_b, stream));
  LCE_LAUNCH("order_extract", stream, launch_order_extract(sort_passes(V) % 2 == 0 ? keys_a : keys_b, V,
                                                   order_dev, stream));
  return LCE_OK;
}

lce_status lce_shard_backward(const void* X_dev, const void* W_shard_dev,
                              const int64_t* labels_dev, const float* lse_dev,
                              const float* dloss_dev, int64_t N, int64_t H, int64_t V_shard,
                              int64_t vocab_offset, int64_t vocab_total, const lce_options* opt,
                              void* dX_part_dev, lce_dtype dX_dtype, void* dW_shard_dev,
                              lce_dtype dW_dtype, void* workspace_dev, size_t workspace_bytes,
                              void* stream_ptr) {
  if (!shape_ok(N, H, V_shard) || !range_ok(V_shard, vocab_offset, vocab_total))
    return LCE_ERR_SHAPE;
  return backward_impl(X_dev, W_shard_dev, labels_dev, lse_dev, dloss_dev, N, H, V_shard,
                       VocabRange{vocab_offset, vocab_total}, nullptr, opt, dX_part_dev, dX_dtype,
                       dW_shard_dev, dW_dtype, workspace_dev, workspace_bytes, stream_ptr);
}

size_t lce_fused_workspace_bytes(int64_t N, int64_t H, int64_t V, lce_dtype dW_dtype) {
  if (!shape_ok(N, H, V) || V > kFusedMaxV || (dW_dtype != LCE_F32 && dW_dtype != LCE_BF16))
    return 0;
  return plan_fused(N, H, V, dW_dtype).total;
}

lce_status lce_forward_backward(const void* X_dev, const void* W_dev, const int64_t* labels_dev,
                                const float* dloss_dev, int64_t N, int64_t H, int64_t V,
                                const lce_options* opt, float* loss_dev, float* lse_dev,
                                float* reduced_dev, int32_t* n_valid_dev, int32_t* bad_label_dev,
                                void* dX_dev, lce_dtype dX_dtype, void* dW_dev,
                                lce_dtype dW_dtype, void* workspace_dev, size_t workspace_bytes,
                                void* stream_ptr) {
  if (!shape_ok(N, H, V) || V > kFusedMaxV) return LCE_ERR_SHAPE;
  if (!options_ok(opt) || !reduced_dev || !n_valid_dev || !dW_dev) return LCE_ERR_INVALID_ARG;
  // Label smoothing needs the softcap derivative apart from the softmax,
  // which the stored logits block does not keep.
  if (opt->label_smoothing > 0.0f && opt->softcap > 0.0f) return LCE_ERR_INVALID_ARG;
  if (opt->filter_eps > 0.0f || opt->precise) return LCE_ERR_INVALID_ARG;
  if ((dX_dtype != LCE_F32 && dX_dtype != LCE_BF16) || (dW_dtype != LCE_F32 && dW_dtype != LCE_BF16))
    return LCE_ERR_INVALID_ARG;
  if (N > 0 && (!X_dev || !W_dev || !labels_dev || !dloss_dev || !loss_dev || !lse_dev ||
                !dX_dev || !workspace_dev))
    return LCE_ERR_INVALID_ARG;
  if (!aligned(X_dev, 16) || !aligned(W_dev, 16) || !aligned(labels_dev, 8) ||
      !aligned(dloss_dev, 4) || !aligned(loss_dev, 4) || !aligned(lse_dev, 4) ||
      !aligned(reduced_dev, 4) || !aligned(n_valid_dev, 4) || !aligned(bad_label_dev, 4) ||
      !aligned(dX_dev, 16) || !aligned(dW_dev, 16) || !aligned(workspace_dev, kAlign))
    return LCE_ERR_ALIGNMENT;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  if (N == 0) {
    LCE_LAUNCH("empty_forward", stream, launch_empty_forward(reduced_dev, n_valid_dev, bad_label_dev, stream));
    LCE_LAUNCH("fill_zero", stream, launch_fill_zero(dW_dev, V * H * (dW_dtype == LCE_BF16 ? 2 : 4), stream));
    return LCE_OK;
  }
  const FusedPlan pl = plan_fused(N, H, V, dW_dtype);
  if (workspace_bytes < pl.total) return LCE_ERR_WORKSPACE;

  int32_t* state = at<int32_t>(workspace_dev, pl.off_state);
  int32_t* key = at<int32_t>(workspace_dev, pl.off_key);
  float* target = at<float>(workspace_dev, pl.off_target);
  float* deriv = at<float>(workspace_dev, pl.off_deriv);
  float* gs = at<float>(workspace_dev, pl.off_gs);
  float* c1 = at<float>(workspace_dev, pl.off_c1);
  float* oh = at<float>(workspace_dev, pl.off_oh);
  float* rrow = at<float>(workspace_dev, pl.off_rrow);
  uint64_t* keys_a = at<uint64_t>(workspace_dev, pl.off_keys_a);
  uint64_t* keys_b = at<uint64_t>(workspace_dev, pl.off_keys_b);
  const uint64_t* keys = sort_passes(N) % 2 == 0 ? keys_a : keys_b;
  float* part_head = at<float>(workspace_dev, pl.off_head);
  float* part_tail = at<float>(workspace_dev, pl.off_tail);
  BlockStats* bprep = at<BlockStats>(workspace_dev, pl.off_bprep);
  BlockStats* bfin = at<BlockStats>(workspace_dev, pl.off_bfin);
  float* scalars = at<float>(workspace_dev, pl.off_scalars);       // [0] a·dloss(/n), [1] = 1
  int32_t* counts = at<int32_t>(workspace_dev, pl.off_scalars + 8);
  float* pm = at<float>(workspace_dev, pl.off_pm);
  float* ps = at<float>(workspace_dev, pl.off_ps);
  float* pz = at<float>(workspace_dev, pl.off_pz);
  uint16_t* U = at<uint16_t>(workspace_dev, pl.off_U);
  float* ref = at<float>(workspace_dev, pl.off_ref);
  uint16_t* Xs = at<uint16_t>(workspace_dev, pl.off_Xs);
  float* dXp = at<float>(workspace_dev, pl.off_dXp);
  float* dW32 = dW_dtype == LCE_F32 ? static_cast<float*>(dW_dev) : at<float>(workspace_dev, pl.off_dWacc);
  float* pcz = at<float>(workspace_dev, pl.off_pcz);
  int32_t* pcb = at<int32_t>(workspace_dev, pl.off_pcb);
  float* lab_dense = at<float>(workspace_dev, pl.off_labd);
  float* lab_oh = at<float>(workspace_dev, pl.off_labo);
  int32_t* dom_col = at<int32_t>(workspace_dev, pl.off_domcol);
  float* dom_coef = at<float>(workspace_dev, pl.off_domc);
  float* de = at<float>(workspace_dev, pl.off_de);
  int32_t* dkey = at<int32_t>(workspace_dev, pl.off_dkey);
  uint64_t* dkeys_a = at<uint64_t>(workspace_dev, pl.off_dkeys_a);
  uint64_t* dkeys_b = at<uint64_t>(workspace_dev, pl.off_dkeys_b);
  const uint64_t* dkeys = sort_passes(N) % 2 == 0 ? dkeys_a : dkeys_b;
  int32_t* dcounts = at<int32_t>(workspace_dev, pl.off_dcounts);
  const uint16_t* X = static_cast<const uint16_t*>(X_dev);
  const uint16_t* W = static_cast<const uint16_t*>(W_dev);
  const bool smoothing = opt->label_smoothing > 0.0f;
  const bool fixed = flce_fixed_reference(opt->softcap);
  const float c2 = opt->softcap * kLog2e;
  const int64_t dx_es = dX_dtype == LCE_BF16 ? 2 : 4;
  // In-place rescale with one scale for every row (no per-row upstream
  // gradient, no Z-loss): G = 2^(ref − lse)·U carries the row's class only, and
  // the scale is applied in fp32 to the dX rows and dW tiles.  Folded into G
  // before its bf16 rounding, it would move a softmax value near 1 off the
  // exactly representable 1.
  const bool unit = !fixed && opt->reduction != LCE_REDUCE_NONE && opt->z_loss == 0.0f;
  const float* post_scale = unit ? scalars : scalars + 1;

  LCE_LAUNCH("row_prep", stream, launch_row_prep(X, W, labels_dev, N, H, V, VocabRange{0, V}, opt->ignore_index,
                          opt->softcap, opt->logit_scale, state, key, target, deriv, bprep, stream));
  LCE_LAUNCH("scale_finalize", stream, launch_scale_finalize(bprep, pl.nb_prep, dloss_dev, opt->reduction == LCE_REDUCE_MEAN,
                                opt->logit_scale, scalars, counts, stream));
  LCE_LAUNCH("sort_by_label", stream, launch_sort_by_label(key, N, keys_a, keys_b, stream));
  const LossTerms terms = loss_terms(opt, V, smoothing ? pz : nullptr);

  for (int c = 0; c < pl.nchunks; ++c) {
    const int64_t r0 = (int64_t)c * pl.Nc;
    const int64_t nr = std::min<int64_t>(pl.Nc, N - r0);
    const int T = (int)ceil_div(nr, kTile);
    FlceParams fp{};
    fp.X = X + r0 * H; fp.W = W; fp.N = nr; fp.H = H; fp.V = V;
    fp.T = T; fp.S = pick_splits(T, pl.n_vtiles); fp.n_vtiles = pl.n_vtiles;
    pick_xcd_grid(fp.T, fp.S, fp.tt, fp.ss);
    fp.softcap = opt->softcap; fp.logit_scale = opt->logit_scale;
    fp.part_m = pm; fp.part_s = ps; fp.part_z = smoothing ? pz : nullptr;
    fp.U = U; fp.ldu = pl.ldu; fp.ref = fixed ? nullptr : ref;
    fp.part_cz = pcz; fp.part_cb = pcb;
    LCE_LAUNCH("flce_logits", stream, launch_flce_logits(fp, stream));
    LCE_LAUNCH("lse_finalize", stream, launch_lse_finalize(pm, ps, fp.S, nr, state + r0, target + r0, terms,
                                lse_dev + r0, loss_dev + r0, bfin + r0 / kTile, nullptr, stream));
    LCE_LAUNCH("row_coef", stream, launch_row_coef(state + r0, lse_dev + r0, deriv + r0,
                            opt->reduction == LCE_REDUCE_NONE ? dloss_dev + r0 : nullptr, scalars, nr,
                            opt->logit_scale, 1.0f - opt->label_smoothing, opt->z_loss, unit, gs + r0,
                            c1 + r0, oh + r0, lab_dense + r0, lab_oh + r0, dom_col + r0, nullptr,
                            stream));
    // The label's entry and a dominant entry of each row leave the stored
    // block and are applied in fp32 (launch_exact_entries), as in the
    // recompute backward.
    ExactParams ep{};
    ep.X = X + r0 * H; ep.W = W; ep.N = nr; ep.H = H; ep.V = V;
    ep.v_begin = 0; ep.chunk_len = V; ep.key_offset = 0; ep.n_vtiles = pl.n_vtiles;
    ep.softcap = opt->softcap; ep.logit_scale = opt->logit_scale;
    ep.lse = lse_dev + r0; ep.row_state = state + r0; ep.row_key = key + r0;
    ep.gs = gs + r0; ep.c1 = c1 + r0;
    ep.eps_over_v = (float)((double)opt->label_smoothing / (double)V);
    ep.one_minus_eps = 1.0f - opt->label_smoothing;
    ep.dom_base = nullptr; ep.cand_z = pcz; ep.cand_b = pcb; ep.cand_splits = fp.S;
    ep.G = U; ep.g_logits = true;
    ep.lab_dense = lab_dense + r0; ep.lab_oh = lab_oh + r0; ep.dom_col = dom_col + r0;
    ep.dom_coef = dom_coef + r0;
    LCE_LAUNCH("exact_entries", stream, launch_exact_entries(ep, stream));
    LCE_LAUNCH("exact_coef", stream, launch_exact_coef(state + r0, key + r0, lab_dense + r0, lab_oh + r0,
                                                      dom_col + r0, dom_coef + r0,
                                                      unit ? scalars : nullptr, nr, oh + r0, de + r0,
                                                      dkey + r0, stream));
    // G = diag(r)·U with the fixed reference (dW from the row-scaled X, dX
    // rows scaled afterwards); otherwise U is turned into G in place.
    if (fixed) {
      LCE_LAUNCH("flce_row_scale", stream, launch_flce_row_scale(X + r0 * H, nr, H, gs + r0, c1 + r0, lse_dev + r0,
                                        c2, rrow + r0, Xs, stream));
    } else {
      LCE_LAUNCH("flce_scale", stream, launch_flce_scale(U, pl.ldu, nr, V, ref, 2 * pl.n_vtiles, c2, lse_dev + r0,
                                    gs + r0, c1 + r0, (float)((double)opt->label_smoothing / (double)V),
                                    stream));
    }
    ChunkGemmParams cp{};
    cp.G = U; cp.ldg = pl.ldu; cp.Wc = W; cp.wc_rows = V; cp.X = fixed ? Xs : X + r0 * H;
    cp.N = nr; cp.H = H; cp.chunk_len = V;
    cp.nt_tok = T; cp.nt_h = pl.nt_h; cp.nt_v = pl.n_vtiles;
    cp.accumulate = 0; cp.dX_acc = dXp; cp.scale = post_scale;
    cp.dW_dst = dW32;
    cp.ksplit = dx_parts(ceil_div(V, kBK), T, pl.nt_h); cp.dx_part_stride = nr * H;
    cp.dw_accumulate = c > 0;
    cp.flags = nullptr;
    LCE_LAUNCH("chunk_gemm", stream, launch_chunk_gemm(cp, stream));
    LCE_LAUNCH("dx_finalize", stream, launch_dx_finalize(dXp, cp.ksplit, nr * H, nr, H, V, state + r0, key + r0, oh + r0, W,
                               post_scale, fixed ? rrow + r0 : nullptr, dom_col + r0, de + r0,
                               nullptr, static_cast<char*>(dX_dev) + r0 * H * dx_es,
                               dX_dtype == LCE_BF16, stream));
  }
  LCE_LAUNCH("mean_finalize", stream, launch_mean_finalize(bfin, (int)ceil_div(N, kTile), opt->reduction == LCE_REDUCE_MEAN,
                                reduced_dev, n_valid_dev, bad_label_dev, stream));
  LCE_LAUNCH("dw_correct", stream, launch_dw_correct(keys, counts, oh, X, N, H, dW32, 0, V, part_head, part_tail, stream));
  LCE_LAUNCH("sort_dominant", stream, launch_sort_by_label(dkey, N, dkeys_a, dkeys_b, stream));
  LCE_LAUNCH("count_dominant", stream, launch_count_keys(dkeys, N, dcounts, stream));
  LCE_LAUNCH("dw_correct", stream, launch_dw_correct(dkeys, dcounts, de, X, N, H, dW32, 0, V, part_head, part_tail, stream));
  if (dW_dtype == LCE_BF16)
    LCE_LAUNCH("cast_bf16", stream, launch_cast_bf16(dW32, static_cast<uint16_t*>(dW_dev), V * H, stream));
  return LCE_OK;
}

}  // extern "C"
