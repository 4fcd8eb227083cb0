/*
 * lce.h — fused LM-head linear + cross-entropy ("linear-LSE") for AMD gfx950.
 *
 * C ABI of liblce.so.  Every pointer argument named *_dev is a device pointer
 * (HIP device memory of the current device); every other pointer is host
 * memory.  All matrices are dense, row-major and contiguous.  The library never
 * allocates or frees memory: the caller owns every buffer, including the
 * workspace, whose size it obtains from the *_workspace_bytes queries.
 *
 * What is computed (sources are web pages, cited by title and section):
 *   z_iv    = x_i · w_v                      logits, never stored
 *             (AI-infra KB page M011, §01: W is [V, D] and Z = H·Wᵀ)
 *   z_iv   <- c·tanh(z_iv / c)              optional logit softcap, c > 0
 *             (Unsloth fused cross-entropy chapter, §4: in-kernel softcap)
 *   LSE_i   = log Σ_v exp(z_iv)             (blog "最贵的一层：深入浅出 Liger
 *             Kernel 与 Cut Cross-Entropy", §三; M011 §03, §05)
 *   loss_i  = LSE_i − z_{i,y_i}, or 0 when y_i == ignore_index
 *             (same blog §三: loss as LSE minus the indexed target logit;
 *             Unsloth chapter §4: label −100 gives 0)
 *   mean    = Σ_i loss_i / n_valid, n_valid = #{i : y_i ≠ ignore_index}
 *             (M011 §04; Unsloth chapter §4, division by n_items)
 *   dZ_iv   = (dloss / n_valid)·(softmax(z_i)_v − [v == y_i])·(1 − tanh²(z_raw/c))
 *             (blog §二/§三: softmax − onehot, recomputed from the saved LSE;
 *             M011 §06; Unsloth chapter §4 for the softcap derivative)
 *   dX      = dZ · W,   dW = dZᵀ · X        (M011 §06)
 *
 * Conventions where the pages leave a choice open:
 *   - labels are already shifted (position i holds the target of row i);
 *   - the LSE of an ignored row is still written; its loss is 0;
 *   - when every row is ignored, mean = 0 and dX = dW = 0;
 *   - a label that is neither ignore_index nor in [0, V) sets the bad-label
 *     flag, gives a NaN loss for that row (so a NaN mean) and NaN gradients;
 *   - results are bitwise reproducible for fixed inputs, shapes and device:
 *     no floating-point atomics are used anywhere.
 *
 * Shapes and alignment (checked on the host before anything is launched):
 *   0 <= N < 2^31 - 1 tokens, 1 <= H < 2^20 with H % 8 == 0, 1 <= V < 2^31 - 1;
 *   X_dev, W_dev, dX_dev, dW_dev must be 16-byte aligned, labels_dev 8-byte,
 *   workspace_dev 256-byte aligned.
 *
 * Streams: every call only enqueues work on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without waiting.  Calls are re-entrant;
 * concurrent calls on different streams need separate workspaces.  The
 * forward and backward calls make no allocation, copy, memset or
 * synchronisation of their own, so they may be captured into a HIP graph on a
 * capturing stream (the upstream-gradient and other inputs must then live in
 * device memory the graph reads at replay).
 */
#ifndef LCE_H_
#define LCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCE_OK = 0,
  LCE_ERR_INVALID_ARG = 1, /* a required pointer is NULL, or an enum is out of range */
  LCE_ERR_SHAPE = 2,       /* N, H or V outside the limits above (H % 8 != 0 included) */
  LCE_ERR_ALIGNMENT = 3,   /* a pointer breaks the alignment rules above */
  LCE_ERR_WORKSPACE = 4,   /* workspace_bytes is below the size the query returns */
  LCE_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed */
  LCE_ERR_SCRATCH_LIMIT = 6 /* lce_forward_noalloc: the shape needs more than the
                               library's fixed scratch (lce_forward_noalloc_max_bytes) */
} lce_status;

typedef enum {
  LCE_F32 = 0,  /* IEEE float32 */
  LCE_BF16 = 1  /* bfloat16, round-to-nearest-even from the float32 result */
} lce_dtype;

/* Workspace (device bytes) lce_forward needs for these sizes; 0 if the shape
 * is invalid.  Pure host computation. */
size_t lce_forward_workspace_bytes(int64_t N, int64_t H, int64_t V);

/* Workspace lce_backward needs.  With dW_dtype == LCE_BF16 the library keeps
 * one float32 vocabulary chunk of dW in the workspace before rounding it. */
size_t lce_backward_workspace_bytes(int64_t N, int64_t H, int64_t V,
                                    lce_dtype dW_dtype);

/*
 * Forward.
 *   X_dev       bf16 [N, H]   hidden states
 *   W_dev       bf16 [V, H]   LM-head weight (lm_head.weight orientation)
 *   labels_dev  int64 [N]     targets in [0, V) or ignore_index
 *   softcap     c > 0 enables z <- c·tanh(z/c); c <= 0 disables it
 * Outputs (all written, none read):
 *   loss_dev    float [N]     per-row loss (0 for ignored rows)
 *   lse_dev     float [N]     per-row log-sum-exp; the only tensor the
 *                             backward needs besides the inputs
 *   mean_dev    float [1]     Σ loss / n_valid (0 when n_valid == 0)
 *   n_valid_dev int32 [1]     number of rows with a target
 *   bad_label_dev int32 [1]   1 if any label is out of range, else 0; may be NULL
 * The N×V logits are never stored; the workspace is O(N) bytes.
 */
lce_status lce_forward(const void* X_dev, const void* W_dev,
                       const int64_t* labels_dev, int64_t N, int64_t H,
                       int64_t V, int64_t ignore_index, float softcap,
                       float* loss_dev, float* lse_dev, float* mean_dev,
                       int32_t* n_valid_dev, int32_t* bad_label_dev,
                       void* workspace_dev, size_t workspace_bytes,
                       void* stream);

/*
 * Backward of the mean loss.
 *   lse_dev     float [N]     LSE written by lce_forward for the same inputs
 *   dloss_dev   float [1]     upstream gradient d(objective)/d(mean)
 *   dX_dev      [N, H] of dX_dtype, overwritten
 *   dW_dev      [V, H] of dW_dtype, overwritten
 * The logits are recomputed tile by tile from X, W and the LSE.  The dense
 * part of dZ is rounded to bf16 for the two gradient contractions, which
 * accumulate in float32; the one-hot part (−1 at the target, times the
 * softcap derivative there) is applied exactly in float32, and so is the
 * scale dloss / n_valid, after the contractions.  Two entries of each row
 * skip the bf16 chunk and are applied in float32 with the one-hot part: the
 * label's, and one whose softmax exceeds 1/2 + 2^-10 if the row has one.
 * The workspace holds one bf16 vocabulary chunk of dZ (never the whole N×V
 * matrix).
 */
lce_status lce_backward(const void* X_dev, const void* W_dev,
                        const int64_t* labels_dev, const float* lse_dev,
                        const float* dloss_dev, int64_t N, int64_t H,
                        int64_t V, int64_t ignore_index, float softcap,
                        void* dX_dev, lce_dtype dX_dtype, void* dW_dev,
                        lce_dtype dW_dtype, void* workspace_dev,
                        size_t workspace_bytes, void* stream);

/*
 * Loss variants.  The AI-infra KB page M011 (§07) lists label smoothing,
 * Z-loss and the reduction mode as terms that need their own definition, and
 * the Unsloth fused cross-entropy chapter (§4) an optional logit scaling next
 * to the softcap.  The definitions taken:
 *   z_iv     = a · (x_i · w_v), then the optional softcap c
 *   loss_i   = LSE_i − (1 − e)·z_{i,y_i} − (e / V)·Σ_v z_iv + l·LSE_i²
 *              (label smoothing e as in PyTorch's CrossEntropyLoss: target
 *              distribution (1 − e)·onehot + e/V; Z-loss l on the row's LSE)
 *   reduced  = Σ_i loss_i / n_valid (MEAN), Σ_i loss_i (SUM, NONE)
 *   dZ_iv    = s_i · a · ((1 + 2l·LSE_i)·softmax_v − (1 − e)·[v == y_i] − e/V)
 *              · (1 − tanh²) with s_i = dloss / n_valid (MEAN), dloss (SUM) or
 *              dloss_i (NONE: one upstream gradient per row).
 * With every option at its default the results are those of lce_forward /
 * lce_backward.
 */
typedef enum {
  LCE_REDUCE_MEAN = 0,
  LCE_REDUCE_SUM = 1,
  LCE_REDUCE_NONE = 2
} lce_reduction;

typedef struct {
  int64_t ignore_index;   /* label value of rows without a target (default −100) */
  float softcap;          /* c > 0 enables z <- c·tanh(z/c) (default 0: off) */
  float logit_scale;      /* a, finite and > 0 (default 1) */
  float label_smoothing;  /* e in [0, 1] (default 0) */
  float z_loss;           /* l, finite and >= 0 (default 0) */
  int32_t reduction;      /* an lce_reduction (default LCE_REDUCE_MEAN) */
  float filter_eps;       /* gradient filter threshold, finite and >= 0 (default 0:
                             exact).  See below. */
  int32_t precise;        /* 1: the softmax part of dZ is carried as two bf16
                             parts (default 0).  See below. */
} lce_options;

/*
 * Gradient filter (opt-in, not exact).  The blog "最贵的一层：深入浅出 Liger
 * Kernel 与 Cut Cross-Entropy" (§三) describes CCE skipping every backward tile
 * whose softmax entries all lie below 2^-12, since in bf16 training such terms
 * vanish in rounding once accumulated; the AI-infra KB page M011 (§06) warns
 * that this drops gradient terms and is separate from the memory saving.
 * With filter_eps > 0, lce_backward_ex and lce_shard_backward skip, in both
 * gradient contractions, every block of 256 token rows by 256 vocabulary
 * columns (aligned to multiples of 256) whose values (1 + 2l·LSE_i)·p_iv over
 * rows with a target all lie below filter_eps.  The recomputation of the
 * logits still runs in full and the one-hot term is always applied exactly.
 * Not combined with label smoothing (LCE_ERR_INVALID_ARG); lce_forward_backward
 * refuses filter_eps > 0; the forward calls ignore it.
 */

/*
 * Precise gradient (opt-in).  The backward carries the softmax part of dZ,
 * softmax·(1 − tanh²) times the row factors, through a bf16 chunk: each value
 * is rounded to 2^-9 of itself.  The label's entry and an entry above half of
 * its row's softmax mass are applied in float32 (they skip the chunk), which
 * keeps ordinary and confident rows far inside the float32 bar; a row whose
 * gradient is carried by a few mid-sized entries (two or three entries near
 * 1/2 or 1/3 of the mass, or a tiny vocabulary) shows the rounding at about
 * 1e-3 relative.  With precise = 1, lce_backward_ex, lce_backward_sorted and
 * lce_shard_backward store each value as hi = bf16(g) and lo = bf16(g − hi)
 * (about 16 significant bits) and run both gradient contractions on each
 * part: the contractions cost twice as much, and the workspace sizes the
 * queries return hold both parts (each vocabulary chunk is half as wide).
 * Not combined with filter_eps > 0 (LCE_ERR_INVALID_ARG); lce_forward_backward
 * refuses it; the forward calls ignore it.  precise must be 0 or 1.
 */

/* Fill *opt with the defaults listed above (host call). */
void lce_options_default(lce_options* opt);

/*
 * Forward with options.  Arguments as lce_forward, plus
 *   opt          host pointer to the options (out-of-range values give
 *                LCE_ERR_INVALID_ARG before anything is launched)
 *   reduced_dev  float [1]  mean (MEAN) or sum (SUM, NONE) of the row losses
 * The workspace size is the one lce_forward_workspace_bytes returns.
 */
lce_status lce_forward_ex(const void* X_dev, const void* W_dev,
                          const int64_t* labels_dev, int64_t N, int64_t H,
                          int64_t V, const lce_options* opt, float* loss_dev,
                          float* lse_dev, float* reduced_dev,
                          int32_t* n_valid_dev, int32_t* bad_label_dev,
                          void* workspace_dev, size_t workspace_bytes,
                          void* stream);

/*
 * Backward with options.  Arguments as lce_backward, plus `opt`; dloss_dev
 * holds one float (MEAN, SUM) or N floats (NONE: the upstream gradient of
 * each row's loss; ignored rows' entries are not used).  The workspace size
 * is the one lce_backward_workspace_bytes returns.  A scale that every row
 * shares (MEAN or SUM without Z-loss) is applied in float32 after the
 * contractions; per-row factors (NONE, Z-loss) are part of the bf16 dZ.
 */
lce_status lce_backward_ex(const void* X_dev, const void* W_dev,
                           const int64_t* labels_dev, const float* lse_dev,
                           const float* dloss_dev, int64_t N, int64_t H,
                           int64_t V, const lce_options* opt, void* dX_dev,
                           lce_dtype dX_dtype, void* dW_dev, lce_dtype dW_dtype,
                           void* workspace_dev, size_t workspace_bytes,
                           void* stream);

/*
 * Vocabulary order for the gradient filter.  The blog "最贵的一层：深入浅出
 * Liger Kernel 与 Cut Cross-Entropy" (§三) pairs CCE's gradient filter with a
 * vocabulary sort: each entry's average logit is recorded, and the backward
 * places the entries that are often large next to each other, so that whole
 * blocks fall below the threshold more often.
 *
 * lce_vocab_order computes, for every entry v, the average of the plain logit
 * x_i·w_v over the rows whose label is not ignore_index (0 for every entry
 * when there is no such row; logit scale and softcap are left out, both being
 * increasing), as w_v·x̄ with x̄ the fp32 mean of those rows, and writes the
 * entries by decreasing average, equal averages by increasing index, NaN
 * averages first.
 *   X_dev, W_dev, labels_dev, N, H, V, ignore_index   as lce_forward
 *   mean_logit_dev  float [V] device, the averages; may be NULL
 *   order_dev       int32 [V] device, order_dev[j] = the entry at position j
 *   workspace       lce_vocab_order_workspace_bytes(N, H, V) bytes, 256-byte
 *                   aligned, caller-owned (0 for an invalid shape)
 * Errors as lce_forward (W_dev and order_dev must not be NULL).  The sums are
 * taken in a fixed order, so the result is reproducible bit for bit.
 */
size_t lce_vocab_order_workspace_bytes(int64_t N, int64_t H, int64_t V);

lce_status lce_vocab_order(const void* X_dev, const void* W_dev,
                           const int64_t* labels_dev, int64_t N, int64_t H,
                           int64_t V, int64_t ignore_index, float* mean_logit_dev,
                           int32_t* order_dev, void* workspace_dev,
                           size_t workspace_bytes, void* stream);

/*
 * Backward on a reordered vocabulary: the result of lce_backward_ex on the
 * vocabulary relabelled by order_dev (position j holds entry order_dev[j];
 * each label moves to its entry's position), with every dW row returned to
 * its entry.  Without the filter this is lce_backward_ex's result up to the
 * order of fp32 additions in dX; with filter_eps > 0 the 256-column blocks of
 * the filter are cut in positions, so an order that gathers the large
 * entries (lce_vocab_order) lets it skip more blocks.
 *   order_dev   int32 [V] device, a permutation of [0, V) (NULL:
 *               LCE_ERR_INVALID_ARG); with entries repeated or out of range
 *               the gradients are undefined, but no memory outside the
 *               arguments and the workspace is touched
 *   workspace   lce_backward_sorted_workspace_bytes(N, H, V, dW_dtype) bytes:
 *               lce_backward_workspace_bytes plus one chunk of W rows (bf16)
 *               and of dW rows (fp32)
 * Other arguments, options and errors as lce_backward_ex.
 */
size_t lce_backward_sorted_workspace_bytes(int64_t N, int64_t H, int64_t V,
                                           lce_dtype dW_dtype);

lce_status lce_backward_sorted(const void* X_dev, const void* W_dev,
                               const int64_t* labels_dev, const float* lse_dev,
                               const float* dloss_dev, int64_t N, int64_t H,
                               int64_t V, const lce_options* opt,
                               const int32_t* order_dev, void* dX_dev,
                               lce_dtype dX_dtype, void* dW_dev, lce_dtype dW_dtype,
                               void* workspace_dev, size_t workspace_bytes,
                               void* stream);

/*
 * Vocabulary shards.  The AI-infra KB page M011 (§07) splits the vocabulary
 * columns over ranks: each row's max, exp-sum and target score must be made
 * global before its loss is formed, the hidden-state gradient is the sum of
 * the shards' contributions, and averaging per-shard cross-entropies is
 * wrong.  The news-site article on GPU acceleration of the loss function
 * (§4.3) describes the same sharded softmax with an all-reduce of the global
 * denominator.  These three calls are the per-rank pieces of that scheme; the
 * exchange between ranks (an all-gather of the [N] partials, an all-reduce of
 * the dX shares) belongs to the caller's collective library.
 *
 * A shard owns the contiguous vocabulary rows [vocab_offset, vocab_offset +
 * V_shard) of a vocabulary of vocab_total rows; W_shard_dev points to those
 * rows (bf16 [V_shard, H]).  Labels are global ids, checked against
 * [0, vocab_total).  Shapes as above, with 0 <= vocab_offset and
 * vocab_offset + V_shard <= vocab_total < 2^31 - 1 (else LCE_ERR_SHAPE).
 */

/*
 * Per-row partials of one shard (workspace: lce_forward_workspace_bytes(N, H,
 * V_shard)).  Only opt's ignore_index, softcap and logit_scale matter here.
 *   lse_part_dev    float [N]  log Σ_{v in shard} exp(z_v)
 *   target_part_dev float [N]  z_{y_i} when the label lies in the shard and the
 *                              row is valid, else 0
 *   zsum_part_dev   float [N]  Σ_{v in shard} z_v; may be NULL (needed by the
 *                              merge only with label smoothing)
 */
lce_status lce_shard_forward(const void* X_dev, const void* W_shard_dev,
                             const int64_t* labels_dev, int64_t N, int64_t H,
                             int64_t V_shard, int64_t vocab_offset,
                             int64_t vocab_total, const lce_options* opt,
                             float* lse_part_dev, float* target_part_dev,
                             float* zsum_part_dev, void* workspace_dev,
                             size_t workspace_bytes, void* stream);

/* Workspace lce_shard_merge needs (O(N / 256) bytes); 0 if N is invalid. */
size_t lce_shard_merge_workspace_bytes(int64_t N);

/*
 * Merge of n_shards shards' partials, laid out [n_shards, N] in shard order
 * (row k·N + i holds shard k's value for row i; zsum_parts_dev may be NULL
 * unless opt->label_smoothing > 0).  LSE_i = m + log Σ_k exp(L_ki − m) with
 * m = max_k L_ki, the target logit and the logit sum are the sums over the
 * shards, each taken in shard order, and the loss, reduction, n_valid and
 * bad-label flag follow lce_forward_ex with vocab_total as V.  Outputs as
 * lce_forward_ex.
 */
lce_status lce_shard_merge(const float* lse_parts_dev, const float* target_parts_dev,
                           const float* zsum_parts_dev, int32_t n_shards,
                           const int64_t* labels_dev, int64_t N, int64_t vocab_total,
                           const lce_options* opt, float* loss_dev, float* lse_dev,
                           float* reduced_dev, int32_t* n_valid_dev,
                           int32_t* bad_label_dev, void* workspace_dev,
                           size_t workspace_bytes, void* stream);

/*
 * Backward of one shard given the merged LSE (workspace:
 * lce_backward_workspace_bytes(N, H, V_shard, dW_dtype)).  dloss_dev as in
 * lce_backward_ex.  The gradient of the shard's logit columns uses the merged
 * LSE; the one-hot term (−(1 − e) at the target) appears only on the shard
 * that owns the label; label smoothing divides by vocab_total.
 *   dX_part_dev  [N, H] of dX_dtype, overwritten: this shard's share of dX
 *                (the shares of all shards add up to dX)
 *   dW_shard_dev [V_shard, H] of dW_dtype, overwritten: rows vocab_offset ...
 *                of dW
 */
lce_status lce_shard_backward(const void* X_dev, const void* W_shard_dev,
                              const int64_t* labels_dev, const float* lse_dev,
                              const float* dloss_dev, int64_t N, int64_t H,
                              int64_t V_shard, int64_t vocab_offset,
                              int64_t vocab_total, const lce_options* opt,
                              void* dX_part_dev, lce_dtype dX_dtype,
                              void* dW_shard_dev, lce_dtype dW_dtype,
                              void* workspace_dev, size_t workspace_bytes,
                              void* stream);

/*
 * Forward and backward in one call, row chunk by row chunk (the FLCE
 * pipeline of Liger: blog "最贵的一层：深入浅出 Liger Kernel 与 Cut
 * Cross-Entropy", §二, and the Liger Kernel paper page, §3.2).  The rows are
 * cut into chunks of whole 256-row tiles, at least one, at most 2H rows and,
 * from two tiles on, at most half the tiles rounded up; as even as whole tiles
 * allow, their count chosen for the least estimated time (lce_fused_plan
 * gives the plan); for each chunk the logits against
 * the whole vocabulary are formed once, kept as a bf16 block of Nc x V in the
 * workspace (at most twice the size of W), turned into the logit
 * gradient, and projected back at once: dX rows = dZ_chunk · W, dW += dZᵀ ·
 * X_chunk.  Three N·H·V contractions instead of the four of lce_forward +
 * lce_backward, for an Nc x V workspace block.
 *
 * Results are those of lce_forward_ex followed by lce_backward_ex with the
 * same options and dloss (within rounding; the stored block adds one bf16
 * rounding of exp(z − ref)·d, like the gradient chunk of lce_backward).
 *   dloss_dev   float [1] (MEAN, SUM) or [N] (NONE), as lce_backward_ex; it is
 *               needed up front because the gradient is formed in the pass
 *   outputs     loss/lse/reduced/n_valid/bad_label as lce_forward_ex, dX and
 *               dW as lce_backward_ex
 * Not supported: label smoothing together with a softcap
 * (LCE_ERR_INVALID_ARG), V > 2^21 (LCE_ERR_SHAPE).  Workspace:
 * lce_fused_workspace_bytes (0 for an invalid shape).
 */
size_t lce_fused_workspace_bytes(int64_t N, int64_t H, int64_t V, lce_dtype dW_dtype);

lce_status lce_forward_backward(const void* X_dev, const void* W_dev,
                                const int64_t* labels_dev, const float* dloss_dev,
                                int64_t N, int64_t H, int64_t V, const lce_options* opt,
                                float* loss_dev, float* lse_dev, float* reduced_dev,
                                int32_t* n_valid_dev, int32_t* bad_label_dev,
                                void* dX_dev, lce_dtype dX_dtype, void* dW_dev,
                                lce_dtype dW_dtype, void* workspace_dev,
                                size_t workspace_bytes, void* stream);

/*
 * Forward without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it).  Same arguments, kernels and results as lce_forward, bit for
 * bit, minus the workspace: the call runs in a scratch array the library
 * holds in device memory, one per device (lce_forward_noalloc_max_bytes()
 * bytes, 64 MiB, held until the process ends).  The array's device address
 * is looked up on the first call on each device.  A shape whose forward
 * workspace (lce_forward_workspace_bytes) exceeds that size returns
 * LCE_ERR_SCRATCH_LIMIT before anything is launched; with the forward's
 * plan that is N above roughly 640 000 rows (V of 2048 or more).  The call
 * itself allocates nothing: no hipMalloc, no host or library allocation on
 * the device.
 * Every call on one device shares that device's array, and each call
 * overwrites it before reading it, so nothing carries over between calls;
 * but calls that overlap in time on one device (concurrent streams, several
 * host threads) race on it and give undefined results.  Serialise them.
 */
size_t lce_forward_noalloc_max_bytes(void);

lce_status lce_forward_noalloc(const void* X_dev, const void* W_dev,
                               const int64_t* labels_dev, int64_t N, int64_t H,
                               int64_t V, int64_t ignore_index, float softcap,
                               float* loss_dev, float* lse_dev, float* mean_dev,
                               int32_t* n_valid_dev, int32_t* bad_label_dev,
                               void* stream);

/*
 * The device a call would run on (host call).  For HIP device `device` (-1:
 * the current device): the number of compute units, the peak shader clock in
 * kHz and the architecture name (NUL-terminated, truncated to arch_len bytes;
 * arch may be NULL).  The dense bf16 MFMA peak of a gfx950 part is
 * cu_count · clock · 4096 flops per clock and compute unit.  Returns LCE_OK,
 * LCE_ERR_INVALID_ARG for NULL outputs, or LCE_ERR_HIP.
 */
lce_status lce_device_info(int device, int32_t* cu_count, int32_t* clock_khz, char* arch,
                           int32_t arch_len);

/*
 * The backward's chunking for these sizes (host call, pure computation, the
 * plan lce_backward and lce_backward_ex follow): the vocabulary columns per
 * bf16 gradient chunk (a multiple of 256; the last chunk may be narrower),
 * the number of chunks, and the K parts the dX tiles of the first chunk are
 * split into (1 when there are enough token tiles; summed in order at the
 * end).  precise (0 or 1) selects the plan of lce_options.precise.  Without
 * the filter and vocabulary order the workspace holds one chunk of
 * 256·ceil(N/256) x chunk_columns bf16 values (twice with precise) and
 * dx_parts fp32 copies of dX.  Returns LCE_OK, LCE_ERR_SHAPE (shape out of
 * range) or LCE_ERR_INVALID_ARG (NULL output, precise not 0 or 1).
 */
lce_status lce_backward_plan(int64_t N, int64_t H, int64_t V, int32_t precise,
                             int64_t* chunk_columns, int32_t* n_chunks, int32_t* dx_parts);

/*
 * The row chunking of lce_forward_backward for these sizes (host call, pure
 * computation, the plan the call follows): the rows per chunk (a multiple of
 * 256; the last chunk holds the rest, at least one row; N = 0 is planned as
 * one row), the number of chunks, and the K parts the dX tiles of a full
 * chunk are split into (a shorter last chunk may take more).  The workspace holds one bf16 block of
 * chunk_rows x 256·ceil(V/256) values.  Returns LCE_OK, LCE_ERR_SHAPE (shape
 * out of range) or LCE_ERR_INVALID_ARG (NULL output).
 */
lce_status lce_fused_plan(int64_t N, int64_t H, int64_t V, int64_t* chunk_rows, int32_t* n_chunks,
                          int32_t* dx_parts);

/* Static, NUL-terminated description of a status code. */
const char* lce_status_string(lce_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lce_version(void);

/*
 * Kernel timing instrumentation (for benchmarks; off by default).
 * While enabled, every kernel the two calls above enqueue is bracketed by a
 * pair of hipEvents recorded on the same stream.  lce_timing_read waits for the
 * recorded events, then fills up to `max_entries` records (one per kernel
 * name, in first-launch order) with the number of launches and their summed
 * duration in milliseconds since the last reset, and returns the number of
 * distinct kernels (which may exceed max_entries).  `out` may be NULL to
 * query the count.  Returns a negative value if a HIP event call failed.
 * Not thread-safe with respect to concurrent lce_forward/lce_backward calls
 * that toggle or read it.
 */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} lce_kernel_timing;

void lce_timing_enable(int enable);
void lce_timing_reset(void);
int lce_timing_read(lce_kernel_timing* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H_ */
