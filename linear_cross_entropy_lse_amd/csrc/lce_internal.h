// Internal interfaces between the liblce entry points and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

// Forward partials of one launch: grid T x S, T token tiles of 256 (at most
// 32 per launch), S vocabulary splits.
struct LseParams {
  const uint16_t* X;  // bf16 [N, H]
  const uint16_t* W;  // bf16 [V, H]
  int64_t N, H, V;
  int T, S, n_vtiles;
  int tt, ss;         // XCD sub-grid (see grid_tile); 0 = plain order
  float softcap;
  float logit_scale;  // a > 0: z = a·(x·w) before the softcap
  float* part_m;      // [S, ldp] base-2 running max
  float* part_s;      // [S, ldp] Σ 2^(u − m)
  float* part_z;      // [S, ldp] Σ_v z_v (label smoothing), or null
  int64_t ldp;        // floats from one split's partials to the next (>= N)
};

// Recomputed logit gradient of one vocabulary chunk [v_begin, v_begin + 256·n_vtiles).
struct GradParams {
  const uint16_t* X;
  const uint16_t* W;
  int64_t N, H, V;
  int64_t v_begin;
  int T, S, n_vtiles;
  int tt, ss;
  int round_tiles;    // > 0: rounds of round_tiles token tiles x S splits (round_tile)
  int t0;             // first token tile of the launch: it covers tiles [t0, t0 + T)
  float softcap;
  float logit_scale;
  const float* lse;          // [N]
  const int32_t* row_state;  // [N]
  // bf16, blocked: block (token tile t, chunk-local vocabulary tile j) at
  // element (t·n_vtiles + j)·65536, as 4 sub-blocks of 256 token rows by 64
  // columns; rows past N hold zeros.  ldg is unused.
  uint16_t* G;
  int64_t ldg;
  // General form (label smoothing, Z-loss, per-row upstream gradient):
  // G = gs_i·(c1_i·p − eps_over_v)·d; null gs selects the plain G = p·d.
  const float* gs;           // [N] per-row scale s_i·a (0 ignored, NaN bad)
  const float* c1;           // [N] 1 + 2l·LSE_i
  float eps_over_v;          // e / V
  // Gradient filter: when flags is not null, byte w of word ti·n_vtiles + j
  // is set to 1 if wave w of tile (ti, j) holds a value of (1 + 2l·LSE)·p,
  // over rows with a target, that is not below filter_eps, else 0.
  uint8_t* flags;
  float filter_eps;
  // Dominant-entry candidates: for the token of a row with an entry whose
  // softmax exceeds 1/2 (at most one per row), the W row of the first of the
  // 64 rows of the tile that the finding lane holds, plus key_offset (rows
  // lrow + x, x < 128 with bit 2 clear); untouched otherwise (the host presets
  // −1).  launch_exact_entries recomputes those 64 logits and keeps the entry
  // if its softmax exceeds 1/2 + 2^-10.
  int32_t* dom_base;
  int64_t key_offset;
  // Precise gradient: when not null, G holds hi = bf16(g) and G_lo, in the
  // same layout, lo = bf16(g − hi).  Not with flags.
  uint16_t* G_lo;
};

// dX and dW contractions of one vocabulary chunk, in one persistent launch of
// kXcds x kCusPerXcd workgroups: nt_tok·nt_h tiles of dX_acc (+)= G · W_chunk
// and nt_v·nt_h tiles of dW_chunk = s·Gᵀ·X.
struct ChunkGemmParams {
  // bf16, blocked (see DtlKMajorBlocked): nt_v blocks of 256 x 256 per token
  // tile, chunk-local vocabulary columns (0 past V), padding rows past N
  // finite.  ldg = 256·nt_v.
  const uint16_t* G;
  int64_t ldg;
  const uint16_t* Wc;  // W + v_begin · H
  int64_t wc_rows;     // V − v_begin (rows of W readable from Wc)
  const uint16_t* X;   // bf16 [N, H]
  int64_t N, H;
  int64_t chunk_len;   // vocabulary rows in this chunk
  int nt_tok, nt_h, nt_v;
  int accumulate;      // 0: first chunk writes dX_acc, 1: later chunks add
  float* dX_acc;       // fp32 [N, H]
  const float* scale;  // device scalar dloss / n_valid
  float* dW_dst;       // fp32 [chunk_len, H] (row v_local)
  // Split of each dX tile's K range (the chunk's vocabulary) into ksplit
  // parts; part k goes to dX_acc + k·dx_part_stride.  1 without splitting.
  int ksplit;
  int64_t dx_part_stride;
  int dw_accumulate;   // 1: dW_dst += s·Gᵀ·X instead of =
  // Gradient filter words [nt_tok, nt_v] (non-zero: the tile's dense part is
  // kept); null: every tile is kept.  Only with ksplit = 1.
  const uint32_t* flags;
};

// Row-chunked forward with the logit gradient formed in the same pass: the
// logits of `N` rows (one chunk) against the whole vocabulary.  Per (token
// tile, split) the (m, s) partials as in LseParams, and every logit as
// U = 2^(u − ref)·d in bf16 ([N, ldu], columns past V written 0), u the
// base-2 (scaled, capped) logit, d the softcap derivative (1 without), ref
// the reference below.
struct FlceParams {
  const uint16_t* X;   // bf16 [N, H] (the chunk's rows)
  const uint16_t* W;   // bf16 [V, H]
  int64_t N, H, V;
  int T, S, n_vtiles;
  int tt, ss;
  float softcap;
  float logit_scale;
  float* part_m;       // [S, N]
  float* part_s;       // [S, N]
  float* part_z;       // [S, N] or null
  uint16_t* U;         // bf16, blocked like ChunkGemmParams::G (n_vtiles blocks per token tile)
  int64_t ldu;         // n_vtiles · 256
  // Reference of each row's 128-column block (base 2), [N, 2·n_vtiles]: the
  // running max of the row's split up to and including that block's tile.
  // Null selects the fixed reference c·log2(e) (softcap with c·log2(e) < 60).
  float* ref;
  // Dominant-entry candidate of each (split, token), [S, N]: the split's
  // largest logit of the token and the W row of the first of the 64 rows of
  // the tile that the lane holding it held (−1: none).
  float* part_cz;
  int32_t* part_cb;
};

hipError_t launch_lse_partials(const LseParams& p, hipStream_t stream);
hipError_t launch_flce_logits(const FlceParams& p, hipStream_t stream);
// True when the fused forward's logits use the fixed reference c·log2(e).
bool flce_fixed_reference(float softcap);
hipError_t launch_grad_logits(const GradParams& p, hipStream_t stream);

// Exact entries of one vocabulary chunk (lce_exact.hip).  Two entries per row
// do not go through the bf16 gradient chunk: the entry at the row's label,
// whose p·d nearly cancels the one-hot term when the row predicts its label
// confidently, and an entry with softmax above 1/2 + 2^-10 (found by the
// logit-gradient pass, dom_base), which alone carries a large share of the
// row's gradient.  For each, the logit is recomputed with the MFMA sequence
// of the tile kernels (so it is the value the forward's LSE and the logit
// gradient saw, bit for bit), its value is written in fp32, and its place in
// the chunk G is overwritten with the value of a logit of −inf (0, or −gs·e/V
// without softcap).  Values in G's units:
//   lab_dense[i]  the label entry minus the −inf value, lab_oh[i] the one-hot
//                 term (1 − e)·d·(gs or 1), for rows whose label (row_key −
//                 key_offset, this call's W rows) lies in the chunk
//   dom_col[i]    the other entry's W row plus key_offset, dom_coef[i] the
//                 entry minus the −inf value, for rows whose dom_base lies in
//                 the chunk (dom_col is preset −1 by the host)
struct ExactParams {
  const uint16_t* X;
  const uint16_t* W;          // this call's W rows (the gathered chunk with an order)
  int64_t N, H, V;            // V: rows of W
  int64_t v_begin, chunk_len; // the chunk's rows of W
  int64_t key_offset;         // row_key − key_offset is a label's row of W
  int n_vtiles;               // vocabulary tiles of the chunk (G layout)
  float softcap, logit_scale;
  const float* lse;
  const int32_t* row_state;
  const int32_t* row_key;
  const float* gs;            // general form (null: plain)
  const float* c1;
  float eps_over_v, one_minus_eps;
  const int32_t* dom_base;
  // Instead of dom_base (null): per-split candidates [cand_splits, N] of the
  // fused forward (FlceParams::part_cz); the best is dominant when its
  // softmax exceeds the threshold.
  const float* cand_z;
  const int32_t* cand_b;
  int cand_splits;
  uint16_t* G;                // blocked chunk, as GradParams::G
  uint16_t* G_lo;             // its lo part (precise gradient), or null
  bool g_logits;              // G holds the fused call's stored logits, turned into the
                              // gradient afterwards by G = f·U − gs·e/V: a taken entry's
                              // slot is then set to 0, whose image is the slot value
  // What the pass does for the label entries (kLabelValues, kLabelSlots or
  // kLabelNone).  kLabelSlots reads the label-sorted keys (row_key << 32 |
  // row, ascending) and the count of rows with a key in range (*n_keys): the
  // rows whose labels fall in this chunk are one run of them.
  int label_pass;
  const uint64_t* keys;
  const int32_t* n_keys;
  float* lab_dense;
  float* lab_oh;
  int32_t* dom_col;
  float* dom_coef;
};
// ExactParams::label_pass: compute the label entries' values (lab_dense,
// lab_oh) of tokens in [v_begin, v_begin + chunk_len), and write the value of
// a logit at −inf into G at them unless G is null; only that write, for the
// labels in this chunk; or nothing.  The dominant-entry part runs when
// dom_base or cand_z is set.
constexpr int kLabelValues = 0, kLabelSlots = 1, kLabelNone = 2;
hipError_t launch_exact_entries(const ExactParams& p, hipStream_t stream);
hipError_t launch_chunk_gemm(const ChunkGemmParams& p, hipStream_t stream);

// Row-wise kernels (lce_rows.hip).
struct BlockStats {  // per-block partial of the row scan, combined in a fixed order
  double loss_sum;
  int32_t n_valid;   // rows with label != ignore_index
  int32_t n_bad;     // ... whose label is outside [0, V_total)
  int32_t n_owned;   // valid rows whose label lies in this call's vocabulary rows
  int32_t pad;
};

// Vocabulary rows a call works on: W holds rows [v_lo, v_lo + V) of a
// vocabulary of V_total rows (v_lo = 0, V_total = V without sharding).
struct VocabRange {
  int64_t v_lo;
  int64_t V_total;
};

// Labels are checked against [0, V_total); a valid row is "owned" when its
// label lies in [v_lo, v_lo + V).  Owned rows get the target logit, its
// softcap derivative and the local label (y − v_lo) as sort key; other rows
// get target 0, derivative 0 and key INT_MAX.
hipError_t launch_row_prep(const uint16_t* X, const uint16_t* W, const int64_t* labels,
                           int64_t N, int64_t H, int64_t V, VocabRange vr, int64_t ignore_index,
                           float softcap, float logit_scale, int32_t* row_state,
                           int32_t* row_key, float* target, float* target_deriv,
                           BlockStats* blocks, hipStream_t stream);
int row_prep_blocks(int64_t N);

// Loss-variant terms applied when the row loss is formed.
struct LossTerms {
  float one_minus_eps;   // 1 − e (target weight)
  float eps_over_v;      // e / V (weight of Σ_v z_v)
  float z_loss;          // l
  const float* part_z;   // [S, N] or null (e = 0)
};

// loss and blocks may be null (a vocabulary shard's partials need neither);
// zsum, when not null, receives the merged Σ_v z_v of each row (needs
// terms.part_z).
hipError_t launch_lse_finalize(const float* part_m, const float* part_s, int S, int64_t N,
                               const int32_t* row_state, const float* target,
                               const LossTerms& terms, float* lse, float* loss,
                               BlockStats* blocks, float* zsum, hipStream_t stream);
int lse_finalize_blocks(int64_t N);

// Merge of g vocabulary shards' row partials, in shard order: lse_parts,
// target_parts and zsum_parts are [g, N] (zsum_parts may be null when
// terms.eps_over_v is 0).  Writes lse, loss and per-block statistics like
// lse_finalize; labels are checked against [0, V_total).
hipError_t launch_shard_merge(const float* lse_parts, const float* target_parts,
                              const float* zsum_parts, int g, const int64_t* labels, int64_t N,
                              int64_t V_total, int64_t ignore_index, const LossTerms& terms,
                              float* lse, float* loss, BlockStats* blocks, hipStream_t stream);

// reduced = Σ loss / n_valid (divide = 1) or Σ loss (divide = 0).
hipError_t launch_mean_finalize(const BlockStats* blocks, int nblocks, int divide, float* reduced,
                                int32_t* n_valid, int32_t* bad_flag, hipStream_t stream);

// scalars[0] = a·dloss / n_valid (divide = 1) or a·dloss (divide = 0), the
// upstream scale of the plain path; scalars[1] = 1.  counts[0] = n_valid,
// counts[1] = owned rows (the rows that get sorted).
hipError_t launch_scale_finalize(const BlockStats* blocks, int nblocks, const float* dloss,
                                 int divide, float logit_scale, float* scalars, int32_t* counts,
                                 hipStream_t stream);

// Per-row gradient coefficients: gs_i (row scale, times a), c1_i = 1 + 2l·LSE_i
// and oh_i = gs_i·(1 − e)·d_i (the one-hot coefficient, d_i the softcap
// derivative at the target).  Row scale: dloss_rows[i] when dloss_rows is not
// null, else the scalar scalars[0] (a included).  unit: the caller applies the
// scalar scalars[0] after the contractions, so gs_i is written as the row's
// class alone (1 valid, 0 ignored, NaN bad); oh_i keeps the full scale.
// lab_dense, lab_oh, dom_col and dom_base, when not null, are preset to 0, 0,
// −1 and −1 for the exact entries (launch_exact_entries).
hipError_t launch_row_coef(const int32_t* row_state, const float* lse, const float* target_deriv,
                           const float* dloss_rows, const float* scalars, int64_t N,
                           float logit_scale, float one_minus_eps, float z_loss, int unit,
                           float* gs, float* c1, float* oh, float* lab_dense, float* lab_oh,
                           int32_t* dom_col, int32_t* dom_base, hipStream_t stream);

// Gradient filter with the exact entries of the vocabulary chunk whose W rows
// are [c_lo, c_lo + 256·n_vt) (in row_key − key_offset space): a row's label
// or dominant dense value is set to 0 when the 256 x 256 block that holds it
// has a zero flag word (skipped), as the block's other dense values are.
hipError_t launch_filter_exact(const uint32_t* flags, int n_vt, int64_t c_lo,
                               const int32_t* row_state, const int32_t* row_key,
                               int64_t key_offset, int64_t N, float* lab_dense,
                               const int32_t* dom_col, float* dom_coef, hipStream_t stream);

// Coefficients of the exact entries for the finalize steps, from the
// logit-gradient pass's per-row outputs: oh[i] = s·(lab_oh[i] − lab_dense[i])
// for rows with a label among this call's W rows (row_state valid, row_key !=
// INT_MAX), else 0; de[i] = −s·dom_coef[i] and dkey[i] = dom_col[i] for rows
// with a dominant entry (dom_col >= 0), else 0 and INT_MAX.  s = scale[0], or
// 1 when scale is null.  (dx_finalize and dw_correct subtract oh·w and oh·x,
// de·w and de·x.)
hipError_t launch_exact_coef(const int32_t* row_state, const int32_t* row_key,
                             const float* lab_dense, const float* lab_oh, const int32_t* dom_col,
                             const float* dom_coef, const float* scale, int64_t N, float* oh,
                             float* de, int32_t* dkey, hipStream_t stream);

// counts[1] = number of sorted keys (of sort_padded(N)) whose label is not
// INT_MAX: the rows launch_dw_correct walks.
hipError_t launch_count_keys(const uint64_t* keys, int64_t N, int32_t* counts, hipStream_t stream);

// Label sort of the valid rows (keys: label << 32 | row, ascending).
constexpr int kSortBlock = 2048;   // keys sorted per block in LDS
int64_t sort_padded(int64_t N);    // N rounded up to kSortBlock
int sort_passes(int64_t N);        // merge passes after the block sort
// Sorted keys end up in keys_a after an even number of passes, else keys_b;
// each buffer holds sort_padded(N) keys.
hipError_t launch_sort_by_label(const int32_t* row_key, int64_t N, uint64_t* keys_a,
                                uint64_t* keys_b, hipStream_t stream);

// dX_i = sx·dX_acc_i − oh_i·w_{key_i} (owned rows), sx·dX_acc_i (valid rows
// whose label lies in another shard), 0 (ignored), NaN (bad).  dX_acc_i is
// the sum of n_parts partial buffers part_stride floats apart, taken in part
// order.  sx is the device scalar sx[0], or sx_rows[i] when sx_rows is not
// null.
// Rows with a dominant entry (dom_col not null, dom_col[i] >= 0) also get
// − de_i·w_{dom_col[i]} (w_{order[dom_col[i]]} when order is not null).
hipError_t launch_dx_finalize(const float* dX_acc, int n_parts, int64_t part_stride, int64_t N,
                              int64_t H, int64_t V, const int32_t* row_state, const int32_t* row_key,
                              const float* oh, const uint16_t* W, const float* sx,
                              const float* sx_rows, const int32_t* dom_col, const float* de,
                              const int32_t* order, void* dX, int dX_bf16, hipStream_t stream);

// Fused forward, generic reference: in place (blocked layout), U[i][v]
// becomes the gradient G = gs_i·(c1_i·U·2^(ref_i,v/128 − lse_i·log2 e) −
// eps_over_v) for rows i < N and v < V, 0 for V <= v < ldu; padding rows stay
// as they are.  ref == null: the fixed reference c2 for every block.
hipError_t launch_flce_scale(uint16_t* U, int64_t ldu, int64_t N, int64_t V, const float* ref,
                             int nref, float c2, const float* lse, const float* gs,
                             const float* c1, float eps_over_v, hipStream_t stream);

// Fused forward, fixed reference: r_i = gs_i·c1_i·2^(c2 − lse_i·log2 e), and
// Xs_i = bf16(r_i·x_i).  The gradient is then G = diag(r)·U, so dW = Uᵀ·Xs
// and dX = diag(r)·(U·W).
hipError_t launch_flce_row_scale(const uint16_t* X, int64_t N, int64_t H, const float* gs,
                                 const float* c1, const float* lse, float c2, float* r,
                                 uint16_t* Xs, hipStream_t stream);

// One-hot part of dW from the sorted keys, in chunks of kSegRows sorted rows;
// part_head / part_tail hold seg_chunks(N) x H floats each.
constexpr int kSegRows = 32;
inline int64_t seg_chunks(int64_t N) { return (N + kSegRows - 1) / kSegRows; }
// dst[v − v_lo] −= Σ_{i : y_i = v} oh_i · x_i for v in [v_lo, v_hi).
hipError_t launch_dw_correct(const uint64_t* keys, const int32_t* counts, const float* oh,
                             const uint16_t* X, int64_t N, int64_t H, float* dst, int64_t v_lo,
                             int64_t v_hi, float* part_head, float* part_tail,
                             hipStream_t stream);

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t count, hipStream_t stream);

// Vocabulary order (lce_order.hip).  Average logit of each entry over the
// rows whose label is not ignore_index: key[v] = w_v·x̄, with x̄ from per-block
// column sums part [mean_row_blocks(N) x H] and row counts cnt; word[v] maps
// key[v] to a 32-bit word in decreasing key order (NaN first), ready for
// launch_sort_by_label.
constexpr int kMeanRows = 256;
inline int64_t mean_row_blocks(int64_t N) { return (N + kMeanRows - 1) / kMeanRows; }
hipError_t launch_vocab_key(const uint16_t* X, const int64_t* labels, int64_t N, int64_t H,
                            const uint16_t* W, int64_t V, int64_t ignore_index, float* part,
                            int32_t* cnt, float* xbar, float* key, uint32_t* word,
                            hipStream_t stream);
// order[j] = low word of the j-th sorted key.
hipError_t launch_order_extract(const uint64_t* keys, int64_t V, int32_t* order,
                                hipStream_t stream);
// pos1[v] = 1 + position of v in order (0: none); pkey[i] = position of the
// label key[i], or INT32_MAX.  pos1 holds V entries rounded up to 16 bytes.
hipError_t launch_position_keys(const int32_t* order, int64_t V, const int32_t* key, int64_t N,
                                int32_t* pos1, int32_t* pkey, hipStream_t stream);
// Wp[j] = W[order[j0 + j]] for j < rows (zero row for an out-of-range entry).
hipError_t launch_gather_rows(const uint16_t* W, int64_t V, int64_t H, const int32_t* order,
                              int64_t j0, int64_t rows, uint16_t* Wp, hipStream_t stream);
// dW[order[j0 + j]] = src[j] (fp32 rows) for j < rows, as fp32 or bf16.
hipError_t launch_scatter_rows(const float* src, int64_t V, int64_t H, const int32_t* order,
                               int64_t j0, int64_t rows, void* dW, int bf16, hipStream_t stream);

hipError_t launch_fill_zero(void* dst, int64_t bytes, hipStream_t stream);

hipError_t launch_empty_forward(float* mean, int32_t* n_valid, int32_t* bad_flag,
                                hipStream_t stream);

}  // namespace lce
