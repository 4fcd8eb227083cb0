// Row-wise kernels of liblce: label classification, the indexed target dot
// product, the fixed-order merge of the forward partials, the mean over valid
// targets, the exact one-hot part of the gradients, and small helpers.
//
// Sources (web pages, by title and section):
//   blog "最贵的一层：深入浅出 Liger Kernel 与 Cut Cross-Entropy", §三: the target
//     logit is one dot product x_i · w_{y_i} per row (an indexed matmul, O(N)
//     output), the loss is LSE minus it.
//   AI-infra KB page M011: §04 sum the per-row losses and divide once by the
//     number of valid targets; §05 merge of (max, sum-exp) partials; §06 the
//     gradient is p − onehot scaled by normalisation and upstream gradient;
//     §07 ignore_index rows contribute nothing.
//   Unsloth fused cross-entropy chapter, §4: label −100 gives loss 0, the
//     softcap derivative 1 − tanh² multiplies the gradient, and the total is
//     divided by n_items, the count of labels ≠ −100.
#include <climits>

#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------
// Row classification and the target logit.  One wave per row.
//   row_state:    0 ignored, 1 valid, 2 label outside [0, V_total)
//   row_key:      y − v_lo for owned rows (valid, label in this call's
//                 vocabulary rows), INT_MAX otherwise (sort key)
//   target:       scaled, softcapped target logit (owned rows), else 0
//   target_deriv: 1 − tanh²(t_raw / c) at the target (1 without softcap) for
//                 owned rows, else 0; t_raw = a·(x_i · w_{y_i})
//   blocks:       per-block counts of non-ignored, bad and owned rows
// ---------------------------------------------------------------------------
constexpr int kRowsPerPrepBlock = 4;

__global__ void __launch_bounds__(256)
row_prep_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                const int64_t* __restrict__ labels, int64_t N, int64_t H, int64_t V,
                VocabRange vr, int64_t ignore_index, float softcap, float logit_scale,
                int32_t* __restrict__ row_state, int32_t* __restrict__ row_key,
                float* __restrict__ target, float* __restrict__ target_deriv,
                BlockStats* __restrict__ blocks) {
  __shared__ int counts[kRowsPerPrepBlock][3];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerPrepBlock + wave;
  int st = kRowIgnored;
  bool owned = false;
  if (row < N) {
    const int64_t y = labels[row];
    st = (y == ignore_index) ? kRowIgnored : ((y >= 0 && y < vr.V_total) ? kRowValid : kRowBad);
    const int64_t yl = y - vr.v_lo;
    owned = st == kRowValid && yl >= 0 && yl < V;
    float t = 0.0f, d = 0.0f;
    if (owned && LCE_DCHECK(H % 8 == 0 && vr.v_lo + V <= vr.V_total)) {
      const uint16_t* xr = X + row * H;
      const uint16_t* wr = W + yl * H;
      float dot = 0.0f;
      for (int64_t c = lane; c < H / 8; c += 64) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + c * 8);
        const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + c * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          dot = fmaf(__uint_as_float(xv[q] << 16), __uint_as_float(wv[q] << 16), dot);
          dot = fmaf(__uint_as_float(xv[q] & 0xffff0000u), __uint_as_float(wv[q] & 0xffff0000u), dot);
        }
      }
      dot = wave_sum(dot) * logit_scale;
      if (softcap > 0.0f) {
        const float th = tanhf(dot / softcap);
        t = softcap * th;
        d = 1.0f - th * th;
      } else {
        t = dot;
        d = 1.0f;
      }
    }
    if (lane == 0) {
      row_state[row] = st;
      if (row_key) row_key[row] = owned ? (int32_t)yl : INT_MAX;
      if (target) target[row] = t;
      if (target_deriv) target_deriv[row] = d;
    }
  }
  if (lane == 0) {
    counts[wave][0] = (st != kRowIgnored);
    counts[wave][1] = (st == kRowBad);
    counts[wave][2] = owned;
  }
  __syncthreads();
  if (threadIdx.x == 0 && blocks) {
    int nv = 0, nb = 0, no = 0;
    for (int w = 0; w < kRowsPerPrepBlock; ++w) {
      nv += counts[w][0];
      nb += counts[w][1];
      no += counts[w][2];
    }
    blocks[blockIdx.x] = BlockStats{0.0, nv, nb, no, 0};
  }
}

int row_prep_blocks(int64_t N) { return (int)((N + kRowsPerPrepBlock - 1) / kRowsPerPrepBlock); }

hipError_t launch_row_prep(const uint16_t* X, const uint16_t* W, const int64_t* labels,
                           int64_t N, int64_t H, int64_t V, VocabRange vr, int64_t ignore_index,
                           float softcap, float logit_scale, int32_t* row_state,
                           int32_t* row_key, float* target, float* target_deriv,
                           BlockStats* blocks, hipStream_t stream) {
  hipLaunchKernelGGL(row_prep_kernel, dim3(row_prep_blocks(N)), dim3(256), 0, stream, X, W,
                     labels, N, H, V, vr, ignore_index, softcap, logit_scale, row_state, row_key,
                     target, target_deriv, blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge the S forward partials of each row in split order, then loss and the
// per-block loss sums (fixed-shape tree in double precision).  With the loss
// variants the row loss is LSE − (1 − e)·t − (e/V)·Σ_v z_v + l·LSE², the
// logit sum merged from its per-split partials in split order.
// ---------------------------------------------------------------------------
constexpr int kFinThreads = 256;

// Loss of one row from its LSE, target logit t and logit sum zs.
__device__ __forceinline__ float row_loss(int st, float lse, float t, float zs,
                                          const LossTerms& terms) {
  if (st == kRowBad) return __builtin_nanf("");
  if (st != kRowValid) return 0.0f;
  float l = fmaf(-terms.one_minus_eps, t, lse);
  if (terms.eps_over_v != 0.0f) l = fmaf(-terms.eps_over_v, zs, l);
  return fmaf(terms.z_loss * lse, lse, l);
}

// Fixed-shape tree over the block's rows; thread 0 stores the block's total.
__device__ void store_block_stats(double lossv, int nv, int nb, BlockStats* __restrict__ blocks) {
  __shared__ double ssum[kFinThreads];
  __shared__ int scnt[kFinThreads][2];
  const int tid = threadIdx.x;
  ssum[tid] = lossv;
  scnt[tid][0] = nv;
  scnt[tid][1] = nb;
  __syncthreads();
  for (int o = kFinThreads / 2; o > 0; o >>= 1) {
    if (tid < o) {
      ssum[tid] += ssum[tid + o];
      scnt[tid][0] += scnt[tid + o][0];
      scnt[tid][1] += scnt[tid + o][1];
    }
    __syncthreads();
  }
  if (tid == 0) blocks[blockIdx.x] = BlockStats{ssum[0], scnt[0][0], scnt[0][1], 0, 0};
}

__global__ void __launch_bounds__(kFinThreads)
lse_finalize_kernel(const float* __restrict__ part_m, const float* __restrict__ part_s, int S,
                    int64_t N, const int32_t* __restrict__ row_state,
                    const float* __restrict__ target, LossTerms terms,
                    float* __restrict__ lse_out, float* __restrict__ loss_out,
                    BlockStats* __restrict__ blocks, float* __restrict__ zsum_out) {
  const int64_t row = (int64_t)blockIdx.x * kFinThreads + threadIdx.x;
  double lossv = 0.0;
  int nv = 0, nb = 0;
  if (row < N) {
    const float NEG_INF = -__builtin_inff();
    float m = NEG_INF;
    for (int s = 0; s < S; ++s) m = fmaxf(m, part_m[(int64_t)s * N + row]);
    float sum = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float ms = part_m[(int64_t)s * N + row];
      if (ms != NEG_INF) sum += part_s[(int64_t)s * N + row] * exp2f(ms - m);
    }
    const float lse = (m + log2f(sum)) * kLn2;
    float zs = 0.0f;
    if (terms.part_z)
      for (int s = 0; s < S; ++s) zs += terms.part_z[(int64_t)s * N + row];
    const int st = row_state[row];
    const float l = row_loss(st, lse, target[row], zs, terms);
    lse_out[row] = lse;
    if (loss_out) loss_out[row] = l;
    if (zsum_out) zsum_out[row] = zs;
    lossv = (double)l;
    nv = st != kRowIgnored;
    nb = st == kRowBad;
  }
  if (blocks) store_block_stats(lossv, nv, nb, blocks);
}

int lse_finalize_blocks(int64_t N) { return (int)((N + kFinThreads - 1) / kFinThreads); }

hipError_t launch_lse_finalize(const float* part_m, const float* part_s, int S, int64_t N,
                               const int32_t* row_state, const float* target,
                               const LossTerms& terms, float* lse, float* loss,
                               BlockStats* blocks, float* zsum, hipStream_t stream) {
  hipLaunchKernelGGL(lse_finalize_kernel, dim3(lse_finalize_blocks(N)), dim3(kFinThreads), 0,
                     stream, part_m, part_s, S, N, row_state, target, terms, lse, loss, blocks,
                     zsum);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge of vocabulary shards (AI-infra KB page M011, §07: with the vocabulary
// split over ranks the max, exp-sum and target score of a row are made global
// before its loss is formed; §05: the (max, sum-exp) merge, here with one
// block per shard).  Shard k reports its row LSE L_k = log Σ_{v in k} e^{z_v}
// (natural log), its target part (the target logit on the owning shard, else
// 0) and its logit sum; they are combined in shard order:
//   LSE = m + log Σ_k e^{L_k − m},  m = max_k L_k;  t = Σ_k t_k;  Σz = Σ_k zs_k.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kFinThreads)
shard_merge_kernel(const float* __restrict__ lse_parts, const float* __restrict__ target_parts,
                   const float* __restrict__ zsum_parts, int g, const int64_t* __restrict__ labels,
                   int64_t N, int64_t V_total, int64_t ignore_index, LossTerms terms,
                   float* __restrict__ lse_out, float* __restrict__ loss_out,
                   BlockStats* __restrict__ blocks) {
  const int64_t row = (int64_t)blockIdx.x * kFinThreads + threadIdx.x;
  double lossv = 0.0;
  int nv = 0, nb = 0;
  if (row < N) {
    const float NEG_INF = -__builtin_inff();
    float m = NEG_INF;
    for (int k = 0; k < g; ++k) m = fmaxf(m, lse_parts[(int64_t)k * N + row]);
    float sum = 0.0f, t = 0.0f, zs = 0.0f;
    for (int k = 0; k < g; ++k) {
      const float lk = lse_parts[(int64_t)k * N + row];
      if (lk != NEG_INF) sum += exp2f((lk - m) * kLog2e);
      t += target_parts[(int64_t)k * N + row];
      if (zsum_parts) zs += zsum_parts[(int64_t)k * N + row];
    }
    const float lse = m == NEG_INF ? NEG_INF : m + log2f(sum) * kLn2;
    const int64_t y = labels[row];
    const int st = (y == ignore_index) ? kRowIgnored
                                       : ((y >= 0 && y < V_total) ? kRowValid : kRowBad);
    const float l = row_loss(st, lse, t, zs, terms);
    lse_out[row] = lse;
    loss_out[row] = l;
    lossv = (double)l;
    nv = st != kRowIgnored;
    nb = st == kRowBad;
  }
  store_block_stats(lossv, nv, nb, blocks);
}

hipError_t launch_shard_merge(const float* lse_parts, const float* target_parts,
                              const float* zsum_parts, int g, const int64_t* labels, int64_t N,
                              int64_t V_total, int64_t ignore_index, const LossTerms& terms,
                              float* lse, float* loss, BlockStats* blocks, hipStream_t stream) {
  hipLaunchKernelGGL(shard_merge_kernel, dim3(lse_finalize_blocks(N)), dim3(kFinThreads), 0,
                     stream, lse_parts, target_parts, zsum_parts, g, labels, N, V_total,
                     ignore_index, terms, lse, loss, blocks);
  return hipGetLastError();
}

// Fixed-order reduction of the block statistics by one workgroup.
__device__ void reduce_blocks(const BlockStats* __restrict__ blocks, int nblocks, double& sum,
                              int& nv, int& nb, int& no) {
  __shared__ double ssum[256];
  __shared__ int scnt[256][3];
  const int tid = threadIdx.x;
  double a = 0.0;
  int v = 0, b = 0, w = 0;
  for (int i = tid; i < nblocks; i += 256) {
    a += blocks[i].loss_sum;
    v += blocks[i].n_valid;
    b += blocks[i].n_bad;
    w += blocks[i].n_owned;
  }
  ssum[tid] = a;
  scnt[tid][0] = v;
  scnt[tid][1] = b;
  scnt[tid][2] = w;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      ssum[tid] += ssum[tid + o];
      scnt[tid][0] += scnt[tid + o][0];
      scnt[tid][1] += scnt[tid + o][1];
      scnt[tid][2] += scnt[tid + o][2];
    }
    __syncthreads();
  }
  sum = ssum[0];
  nv = scnt[0][0];
  nb = scnt[0][1];
  no = scnt[0][2];
}

__global__ void __launch_bounds__(256)
mean_finalize_kernel(const BlockStats* __restrict__ blocks, int nblocks, int divide,
                     float* reduced, int32_t* n_valid, int32_t* bad_flag) {
  double sum;
  int nv, nb, no;
  reduce_blocks(blocks, nblocks, sum, nv, nb, no);
  if (threadIdx.x == 0) {
    if (divide) *reduced = nv > 0 ? (float)(sum / (double)nv) : 0.0f;
    else *reduced = (float)sum;
    *n_valid = nv;
    if (bad_flag) *bad_flag = nb > 0 ? 1 : 0;
  }
}

hipError_t launch_mean_finalize(const BlockStats* blocks, int nblocks, int divide, float* reduced,
                                int32_t* n_valid, int32_t* bad_flag, hipStream_t stream) {
  hipLaunchKernelGGL(mean_finalize_kernel, dim3(1), dim3(256), 0, stream, blocks, nblocks, divide,
                     reduced, n_valid, bad_flag);
  return hipGetLastError();
}

// scalars[0] = a·dloss / n_valid (divide; 0 when no row has a target) or
// a·dloss, the upstream scale of the plain gradient path; scalars[1] = 1.
// counts[0] = n_valid, counts[1] = owned rows (valid, label among this call's
// vocabulary rows: the rows that get sorted).
__global__ void __launch_bounds__(256)
scale_finalize_kernel(const BlockStats* __restrict__ blocks, int nblocks,
                      const float* __restrict__ dloss, int divide, float logit_scale,
                      float* scalars, int32_t* counts) {
  double sum;
  int nv, nb, no;
  reduce_blocks(blocks, nblocks, sum, nv, nb, no);
  if (threadIdx.x == 0) {
    const float base = divide ? (nv > 0 ? __fdiv_rn(*dloss, (float)nv) : 0.0f) : *dloss;
    scalars[0] = base * logit_scale;
    scalars[1] = 1.0f;
    counts[0] = nv;
    counts[1] = no;
  }
}

hipError_t launch_scale_finalize(const BlockStats* blocks, int nblocks, const float* dloss,
                                 int divide, float logit_scale, float* scalars, int32_t* counts,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(scale_finalize_kernel, dim3(1), dim3(256), 0, stream, blocks, nblocks,
                     dloss, divide, logit_scale, scalars, counts);
  return hipGetLastError();
}

// Per-row coefficients of the gradient (see launch_row_coef).
__global__ void __launch_bounds__(256)
row_coef_kernel(const int32_t* __restrict__ row_state, const float* __restrict__ lse,
                const float* __restrict__ target_deriv, const float* __restrict__ dloss_rows,
                const float* __restrict__ scalars, int64_t N, float logit_scale,
                float one_minus_eps, float z_loss, int unit, float* __restrict__ gs,
                float* __restrict__ c1, float* __restrict__ oh, float* __restrict__ lab_dense,
                float* __restrict__ lab_oh, int32_t* __restrict__ dom_col,
                int32_t* __restrict__ dom_base) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  if (lab_dense) lab_dense[i] = 0.0f;
  if (lab_oh) lab_oh[i] = 0.0f;
  if (dom_col) dom_col[i] = -1;
  if (dom_base) dom_base[i] = -1;
  const int st = row_state[i];
  float g = 0.0f;
  if (st == kRowValid) g = dloss_rows ? dloss_rows[i] * logit_scale : scalars[0];
  else if (st == kRowBad) g = __builtin_nanf("");
  if (gs) gs[i] = unit ? (st == kRowValid ? 1.0f : (st == kRowBad ? __builtin_nanf("") : 0.0f)) : g;
  if (c1) c1[i] = fmaf(2.0f * z_loss, lse[i], 1.0f);
  oh[i] = st == kRowValid ? g * one_minus_eps * target_deriv[i] : 0.0f;
}

hipError_t launch_row_coef(const int32_t* row_state, const float* lse, const float* target_deriv,
                           const float* dloss_rows, const float* scalars, int64_t N,
                           float logit_scale, float one_minus_eps, float z_loss, int unit,
                           float* gs, float* c1, float* oh, float* lab_dense, float* lab_oh,
                           int32_t* dom_col, int32_t* dom_base, hipStream_t stream) {
  hipLaunchKernelGGL(row_coef_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream,
                     row_state, lse, target_deriv, dloss_rows, scalars, N, logit_scale,
                     one_minus_eps, z_loss, unit, gs, c1, oh, lab_dense, lab_oh, dom_col, dom_base);
  return hipGetLastError();
}

// Filtered blocks and the exact entries (see launch_filter_exact).
__global__ void __launch_bounds__(256)
filter_exact_kernel(const uint32_t* __restrict__ flags, int n_vt, int64_t c_lo,
                    const int32_t* __restrict__ row_state, const int32_t* __restrict__ row_key,
                    int64_t key_offset, int64_t N, float* __restrict__ lab_dense,
                    const int32_t* __restrict__ dom_col, float* __restrict__ dom_coef) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N || row_state[i] != kRowValid) return;
  const int64_t c_hi = c_lo + (int64_t)n_vt * 256;
  const uint32_t* fr = flags + (i / 256) * n_vt;     // the row's token tile
  const int32_t key = row_key[i];
  if (key != INT_MAX) {
    const int64_t L = (int64_t)key - key_offset;
    if (L >= c_lo && L < c_hi && fr[(L - c_lo) / 256] == 0u) lab_dense[i] = 0.0f;
  }
  const int32_t dc = dom_col[i];
  if (dc >= 0) {
    const int64_t L = (int64_t)dc - key_offset;
    if (L >= c_lo && L < c_hi && fr[(L - c_lo) / 256] == 0u) dom_coef[i] = 0.0f;
  }
}

hipError_t launch_filter_exact(const uint32_t* flags, int n_vt, int64_t c_lo,
                               const int32_t* row_state, const int32_t* row_key,
                               int64_t key_offset, int64_t N, float* lab_dense,
                               const int32_t* dom_col, float* dom_coef, hipStream_t stream) {
  hipLaunchKernelGGL(filter_exact_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream,
                     flags, n_vt, c_lo, row_state, row_key, key_offset, N, lab_dense, dom_col,
                     dom_coef);
  return hipGetLastError();
}

// Coefficients of the exact entries (see launch_exact_coef).
__global__ void __launch_bounds__(256)
exact_coef_kernel(const int32_t* __restrict__ row_state, const int32_t* __restrict__ row_key,
                  const float* __restrict__ lab_dense, const float* __restrict__ lab_oh,
                  const int32_t* __restrict__ dom_col, const float* __restrict__ dom_coef,
                  const float* __restrict__ scale, int64_t N, float* __restrict__ oh,
                  float* __restrict__ de, int32_t* __restrict__ dkey) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const float s = scale ? *scale : 1.0f;
  const bool owned = row_state[i] == kRowValid && row_key[i] != INT_MAX;
  oh[i] = owned ? s * (lab_oh[i] - lab_dense[i]) : 0.0f;
  const int32_t c = dom_col[i];
  de[i] = c >= 0 ? -s * dom_coef[i] : 0.0f;
  dkey[i] = c >= 0 ? c : INT_MAX;
}

hipError_t launch_exact_coef(const int32_t* row_state, const int32_t* row_key,
                             const float* lab_dense, const float* lab_oh, const int32_t* dom_col,
                             const float* dom_coef, const float* scale, int64_t N, float* oh,
                             float* de, int32_t* dkey, hipStream_t stream) {
  hipLaunchKernelGGL(exact_coef_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, stream,
                     row_state, row_key, lab_dense, lab_oh, dom_col, dom_coef, scale, N, oh, de,
                     dkey);
  return hipGetLastError();
}

// First sorted key whose label is INT_MAX (binary search; keys ascending).
__global__ void count_keys_kernel(const uint64_t* __restrict__ keys, int64_t n,
                                  int32_t* __restrict__ counts) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int32_t)(keys[mid] >> 32) != INT_MAX && keys[mid] != ~0ull) lo = mid + 1;
    else hi = mid;
  }
  counts[1] = (int32_t)lo;
}

hipError_t launch_count_keys(const uint64_t* keys, int64_t N, int32_t* counts, hipStream_t stream) {
  hipLaunchKernelGGL(count_keys_kernel, dim3(1), dim3(1), 0, stream, keys, sort_padded(N), counts);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Order of the valid rows by label, ties in row order: a sort of the unique
// 64-bit keys (label << 32 | row).  Rows without an in-range label carry the
// label INT_MAX and padding carries ~0, so both end up behind every valid row.
// Step 1 sorts blocks of kSortBlock keys in LDS (bitonic network); step 2
// merges sorted runs pairwise (each output element finds its source by a
// binary search along the merge path), doubling the run length per pass.
// ---------------------------------------------------------------------------
// One thread per compare pair (kSortBlock / 2 threads), so each of the
// network's stages is one exchange and one barrier.
constexpr int kSortThreads = kSortBlock / 2;

__global__ void __launch_bounds__(kSortThreads)
sort_block_kernel(const int32_t* __restrict__ row_key, int64_t N, uint64_t* __restrict__ out) {
  __shared__ uint64_t sk[kSortBlock];
  const int64_t base = (int64_t)blockIdx.x * kSortBlock;
  for (int i = threadIdx.x; i < kSortBlock; i += kSortThreads) {
    const int64_t row = base + i;
    sk[i] = row < N ? ((uint64_t)(uint32_t)row_key[row] << 32) | (uint64_t)row : ~0ull;
  }
  __syncthreads();
  const int t = threadIdx.x;   // compare pair t
  for (int k = 2; k <= kSortBlock; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int i = 2 * t - (t & (j - 1));   // its lower element
      const uint64_t a = sk[i], b = sk[i + j];
      if ((a > b) == ((i & k) == 0)) {
        sk[i] = b;
        sk[i + j] = a;
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < kSortBlock; i += kSortThreads) out[base + i] = sk[i];
}

__global__ void __launch_bounds__(256)
merge_pass_kernel(const uint64_t* __restrict__ in, uint64_t* __restrict__ out, int64_t n,
                  int64_t run) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n) return;
  const int64_t q0 = g / (2 * run) * (2 * run);
  const int64_t lenA = run < n - q0 ? run : n - q0;
  const int64_t b0 = q0 + lenA;
  const int64_t lenB = b0 >= n ? 0 : (run < n - b0 ? run : n - b0);
  const int64_t o = g - q0;
  int64_t lo = o - lenB > 0 ? o - lenB : 0, hi = o < lenA ? o : lenA;
  while (lo < hi) {   // smallest a with A[a] not before B[o − a − 1]
    const int64_t mid = (lo + hi) >> 1;
    if (in[q0 + mid] < in[b0 + o - mid - 1]) lo = mid + 1;
    else hi = mid;
  }
  const int64_t a = lo, b = o - lo;
  const uint64_t v = (b >= lenB || (a < lenA && in[q0 + a] < in[b0 + b])) ? in[q0 + a] : in[b0 + b];
  out[g] = v;
}

int64_t sort_padded(int64_t N) { return (N + kSortBlock - 1) / kSortBlock * kSortBlock; }

int sort_passes(int64_t N) {
  int passes = 0;
  for (int64_t run = kSortBlock; run < sort_padded(N); run *= 2) ++passes;
  return passes;
}

hipError_t launch_sort_by_label(const int32_t* row_key, int64_t N, uint64_t* keys_a,
                                uint64_t* keys_b, hipStream_t stream) {
  const int64_t n = sort_padded(N);
  const int passes = sort_passes(N);
  hipLaunchKernelGGL(sort_block_kernel, dim3((unsigned)(n / kSortBlock)), dim3(kSortThreads), 0, stream,
                     row_key, N, keys_a);
  uint64_t* src = keys_a;
  uint64_t* dst = keys_b;
  int64_t run = kSortBlock;
  for (int ps = 0; ps < passes; ++ps, run *= 2) {
    hipLaunchKernelGGL(merge_pass_kernel, dim3((unsigned)(n / 256)), dim3(256), 0, stream, src, dst, n,
                       run);
    uint64_t* t = src;
    src = dst;
    dst = t;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dX_i = sx · dX_acc[i] − oh_i · w_{y_i}   (valid rows)
//      = 0 (ignored rows), NaN (bad rows)
// The one-hot part of dZ (coefficient oh_i at the target) is applied here
// exactly in fp32; sx is the upstream scale when G was stored unscaled, 1
// when G already carries each row's scale.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
dx_finalize_kernel(const float* __restrict__ dX_acc, int n_parts, int64_t part_stride, int64_t N,
                   int64_t H, int64_t V, const int32_t* __restrict__ row_state,
                   const int32_t* __restrict__ row_key, const float* __restrict__ oh,
                   const uint16_t* __restrict__ W, const float* __restrict__ sx,
                   const float* __restrict__ sx_rows, const int32_t* __restrict__ dom_col,
                   const float* __restrict__ de, const int32_t* __restrict__ order,
                   void* __restrict__ dX, int dX_bf16) {
  const int64_t row = blockIdx.x;
  const int st = row_state[row];
  const float s = sx_rows ? sx_rows[row] : *sx;
  const float e = oh[row];
  const int32_t key = st == kRowValid ? row_key[row] : INT_MAX;
  const bool owned = key != INT_MAX && LCE_DCHECK(key >= 0 && key < V);  // the label is one of W's rows
  const int64_t y = owned ? key : 0;
  const int32_t dc = (dom_col && st == kRowValid) ? dom_col[row] : -1;
  const int64_t yd = dc >= 0 ? (order ? order[dc] : dc) : 0;
  const bool dom = dc >= 0 && LCE_DCHECK(dc < V && yd >= 0 && yd < V);  // a dominant entry other than the label
  const float ed = dom ? de[row] : 0.0f;
  for (int64_t h = (int64_t)threadIdx.x * 4; h < H; h += 1024) {
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (st == kRowValid) {
      float4 v = *reinterpret_cast<const float4*>(dX_acc + row * H + h);
      for (int k = 1; k < n_parts; ++k) {
        const float4 w = *reinterpret_cast<const float4*>(dX_acc + k * part_stride + row * H + h);
        v.x += w.x;
        v.y += w.y;
        v.z += w.z;
        v.w += w.w;
      }
      const float a[4] = {v.x, v.y, v.z, v.w};
      float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // the exact terms, − e·w_y − ed·w_yd
      if (owned) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(W + y * H + h);
        const float w4[4] = {__uint_as_float(wv[0] << 16), __uint_as_float(wv[0] & 0xffff0000u),
                             __uint_as_float(wv[1] << 16), __uint_as_float(wv[1] & 0xffff0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = -e * w4[q];
      }
      if (dom) {
        const u32x2 wv = *reinterpret_cast<const u32x2*>(W + yd * H + h);
        const float w4[4] = {__uint_as_float(wv[0] << 16), __uint_as_float(wv[0] & 0xffff0000u),
                             __uint_as_float(wv[1] << 16), __uint_as_float(wv[1] & 0xffff0000u)};
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = fmaf(-ed, w4[q], t[q]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = fmaf(s, a[q], t[q]);
    } else if (st == kRowBad) {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __builtin_nanf("");
    }
    if (dX_bf16) {
      u32x2 pk;
      pk[0] = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
      pk[1] = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dX) + row * H + h) = pk;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(dX) + row * H + h) =
          make_float4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_dx_finalize(const float* dX_acc, int n_parts, int64_t part_stride, int64_t N,
                              int64_t H, int64_t V, const int32_t* row_state, const int32_t* row_key,
                              const float* oh, const uint16_t* W, const float* sx,
                              const float* sx_rows, const int32_t* dom_col, const float* de,
                              const int32_t* order, void* dX, int dX_bf16, hipStream_t stream) {
  hipLaunchKernelGGL(dx_finalize_kernel, dim3((unsigned)N), dim3(256), 0, stream, dX_acc, n_parts,
                     part_stride, N, H, V, row_state, row_key, oh, W, sx, sx_rows, dom_col, de, order,
                     dX, dX_bf16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused row-chunk variant: turn the stored U = 2^(u − ref)·d of a chunk into
// the logit gradient (see launch_flce_scale).  U is blocked: each thread takes
// 16 consecutive bytes, 8 columns of one token row inside a 64-column
// sub-block, so one reference (one exponential) serves a thread.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
flce_scale_kernel(uint16_t* __restrict__ U, int64_t nvt, int64_t N, int64_t V, int64_t total,
                  const float* __restrict__ ref, int nref, float c2,
                  const float* __restrict__ lse, const float* __restrict__ gs,
                  const float* __restrict__ c1, float eps_over_v) {
  const int64_t o = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (o >= total) return;
  const int64_t blk = o / 65536, rem = o % 65536;
  const int64_t row = blk / nvt * 256 + (rem % 16384) / 64;
  if (row >= N) return;
  const int64_t col0 = blk % nvt * 256 + rem / 16384 * 64 + rem % 64;
  const float g = gs[row];
  const float r = ref ? ref[row * nref + col0 / 128] : c2;
  const float f = g * c1[row] * exp2f(r - lse[row] * kLog2e);
  const float eb = g * eps_over_v;
  uint16_t* p = U + o;
  const u32x4 in = *reinterpret_cast<const u32x4*>(p);
  u32x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = fmaf(f, __uint_as_float(in[q] << 16), -eb);
    const float hi = fmaf(f, __uint_as_float(in[q] & 0xffff0000u), -eb);
    const bool ok_lo = col0 + 2 * q < V, ok_hi = col0 + 2 * q + 1 < V;
    out[q] = pack_bf16x2(ok_lo ? lo : 0.0f, ok_hi ? hi : 0.0f);
  }
  *reinterpret_cast<u32x4*>(p) = out;
}

hipError_t launch_flce_scale(uint16_t* U, int64_t ldu, int64_t N, int64_t V, const float* ref,
                             int nref, float c2, const float* lse, const float* gs,
                             const float* c1, float eps_over_v, hipStream_t stream) {
  const int64_t nvt = ldu / 256;
  const int64_t total = (N + 255) / 256 * 256 * ldu;
  const int64_t threads = total / 8;
  hipLaunchKernelGGL(flce_scale_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, U, nvt, N, V, total, ref, nref, c2, lse, gs, c1, eps_over_v);
  return hipGetLastError();
}

// Fixed-reference form: r_i = gs_i·c1_i·2^(c2 − lse_i·log2 e), Xs_i = bf16(r_i·x_i).
__global__ void __launch_bounds__(256)
flce_row_scale_kernel(const uint16_t* __restrict__ X, int64_t H, const float* __restrict__ gs,
                      const float* __restrict__ c1, const float* __restrict__ lse, float c2,
                      float* __restrict__ r_out, uint16_t* __restrict__ Xs) {
  const int64_t row = blockIdx.x;
  const float r = gs[row] * c1[row] * exp2f(c2 - lse[row] * kLog2e);
  if (threadIdx.x == 0) r_out[row] = r;
  for (int64_t h = (int64_t)threadIdx.x * 8; h < H; h += 256 * 8) {
    const u32x4 in = *reinterpret_cast<const u32x4*>(X + row * H + h);
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      out[q] = pack_bf16x2(r * __uint_as_float(in[q] << 16),
                           r * __uint_as_float(in[q] & 0xffff0000u));
    *reinterpret_cast<u32x4*>(Xs + row * H + h) = out;
  }
}

hipError_t launch_flce_row_scale(const uint16_t* X, int64_t N, int64_t H, const float* gs,
                                 const float* c1, const float* lse, float c2, float* r,
                                 uint16_t* Xs, hipStream_t stream) {
  hipLaunchKernelGGL(flce_row_scale_kernel, dim3((unsigned)N), dim3(256), 0, stream, X, H, gs, c1,
                     lse, c2, r, Xs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dW_v −= Σ_{i : y_i = v} oh_i · x_i for every label v in [v_lo, v_hi)
// (dst row v − v_lo), from the label-sorted keys; oh_i is the one-hot
// coefficient of row i (upstream scale included).
//
// dw_seg_kernel: block (c, slice) walks sorted positions [32c, 32c + 32) in
// order, 8 columns per lane, accumulating one run of equal labels at a time.
// A run that starts and ends inside the chunk is applied at once; the run at
// the chunk start that continues from the previous chunk goes to
// part_head[c]; a run that starts in the chunk and continues into the next
// goes to part_tail[c].  dw_seg_fix_kernel then adds, for each such run,
// part_tail of its first chunk and part_head of every later chunk it covers,
// in chunk order, and applies the total.  Every sum is taken in a fixed
// order, so the result is reproducible bit for bit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t key_label(uint64_t k) { return (int32_t)(k >> 32); }

__global__ void __launch_bounds__(64)
dw_seg_kernel(const uint64_t* __restrict__ keys, const int32_t* __restrict__ counts,
              const float* __restrict__ oh, const uint16_t* __restrict__ X, int64_t n_rows,
              int64_t H, float* __restrict__ dst, int64_t v_lo, int64_t v_hi,
              float* __restrict__ part_head, float* __restrict__ part_tail) {
  __shared__ int32_t s_row[kSegRows], s_lab[kSegRows];
  __shared__ float s_e[kSegRows];
  const int64_t n_ok = counts[1];
  const int64_t c = blockIdx.x;
  const int64_t p0 = c * kSegRows;
  if (p0 >= n_ok) return;
  const int cnt = (int)(n_ok - p0 < kSegRows ? n_ok - p0 : kSegRows);
  const int lane = threadIdx.x;
  if (lane < cnt) {
    const uint64_t k = keys[p0 + lane];
    const bool ok = LCE_DCHECK((int64_t)(uint32_t)k < n_rows);
    s_row[lane] = ok ? (int32_t)(uint32_t)k : 0;
    s_lab[lane] = key_label(k);
    s_e[lane] = ok ? oh[(uint32_t)k] : 0.0f;
  }
  const int32_t lab_prev = p0 > 0 ? key_label(keys[p0 - 1]) : -1;
  const int32_t lab_next = p0 + cnt < n_ok ? key_label(keys[p0 + cnt]) : -1;
  __syncthreads();
  const int64_t h = (int64_t)blockIdx.y * 512 + lane * 8;
  const bool col_ok = h < H;
  // All rows of the chunk are loaded up front so the loads overlap.
  u32x4 xv[kSegRows];
#pragma unroll
  for (int i = 0; i < kSegRows; ++i)
    xv[i] = (col_ok && i < cnt) ? *reinterpret_cast<const u32x4*>(X + (int64_t)s_row[i] * H + h)
                                : u32x4{0u, 0u, 0u, 0u};
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int run_start = 0;
#pragma unroll
  for (int i = 0; i < kSegRows; ++i) {
    if (i < cnt) {
      const float e = s_e[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = fmaf(e, __uint_as_float(xv[i][k] << 16), acc[2 * k]);
        acc[2 * k + 1] = fmaf(e, __uint_as_float(xv[i][k] & 0xffff0000u), acc[2 * k + 1]);
      }
      const int32_t v = s_lab[i];
      if (i + 1 == cnt || s_lab[i + 1] != v) {      // last row of this run
        const bool open_left = run_start == 0 && lab_prev == v;
        const bool open_right = i + 1 == cnt && lab_next == v;
        if (col_ok) {
          if (open_left || open_right) {
            float* d = (open_left ? part_head : part_tail) + c * H + h;
#pragma unroll
            for (int k = 0; k < 8; ++k) d[k] = acc[k];
          } else if (v >= v_lo && v < v_hi) {
            float* d = dst + (int64_t)(v - v_lo) * H + h;
#pragma unroll
            for (int k = 0; k < 8; ++k) d[k] -= acc[k];
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
        run_start = i + 1;
      }
    }
  }
}

__global__ void __launch_bounds__(64)
dw_seg_fix_kernel(const uint64_t* __restrict__ keys, const int32_t* __restrict__ counts, int64_t H,
                  float* __restrict__ dst, int64_t v_lo, int64_t v_hi,
                  const float* __restrict__ part_head, const float* __restrict__ part_tail) {
  const int64_t n_ok = counts[1];
  const int64_t c = blockIdx.x;
  const int64_t p0 = c * kSegRows;
  if (p0 >= n_ok) return;
  const int64_t p1 = p0 + kSegRows < n_ok ? p0 + kSegRows : n_ok;
  const int32_t v = key_label(keys[p1 - 1]);
  if (p1 >= n_ok || key_label(keys[p1]) != v) return;           // last run ends in this chunk
  if (key_label(keys[p0]) == v && p0 > 0 && key_label(keys[p0 - 1]) == v) return;  // not its first chunk
  if (v < v_lo || v >= v_hi) return;
  const int64_t h = (int64_t)blockIdx.y * 512 + threadIdx.x * 8;
  if (h >= H) return;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = part_tail[c * H + h + k];
  for (int64_t c2 = c + 1;; ++c2) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += part_head[c2 * H + h + k];
    const int64_t q0 = c2 * kSegRows;
    const int64_t q1 = q0 + kSegRows < n_ok ? q0 + kSegRows : n_ok;
    if (!(q1 < n_ok && key_label(keys[q1 - 1]) == v && key_label(keys[q1]) == v)) break;
  }
  float* d = dst + (int64_t)(v - v_lo) * H + h;
#pragma unroll
  for (int k = 0; k < 8; ++k) d[k] -= acc[k];
}

hipError_t launch_dw_correct(const uint64_t* keys, const int32_t* counts, const float* oh,
                             const uint16_t* X, int64_t N, int64_t H, float* dst, int64_t v_lo,
                             int64_t v_hi, float* part_head, float* part_tail,
                             hipStream_t stream) {
  const dim3 grid((unsigned)seg_chunks(N), (unsigned)((H + 511) / 512));
  hipLaunchKernelGGL(dw_seg_kernel, grid, dim3(64), 0, stream, keys, counts, oh, X, N, H, dst,
                     v_lo, v_hi, part_head, part_tail);
  hipLaunchKernelGGL(dw_seg_fix_kernel, grid, dim3(64), 0, stream, keys, counts, H, dst, v_lo,
                     v_hi, part_head, part_tail);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
__global__ void cast_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                 int64_t count4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    u32x2 pk;
    pk[0] = f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16);
    pk[1] = f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16);
    reinterpret_cast<u32x2*>(dst)[i] = pk;
  }
}

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, int64_t count, hipStream_t stream) {
  const int64_t n4 = count / 4;
  int64_t grid = (n4 + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, src, dst, n4);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(u32x4* __restrict__ dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t launch_fill_zero(void* dst, int64_t bytes, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  int64_t grid = (n16 + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

__global__ void empty_forward_kernel(float* mean, int32_t* n_valid, int32_t* bad_flag) {
  *mean = 0.0f;
  *n_valid = 0;
  if (bad_flag) *bad_flag = 0;
}

hipError_t launch_empty_forward(float* mean, int32_t* n_valid, int32_t* bad_flag,
                                hipStream_t stream) {
  hipLaunchKernelGGL(empty_forward_kernel, dim3(1), dim3(1), 0, stream, mean, n_valid, bad_flag);
  return hipGetLastError();
}

}  // namespace lce
