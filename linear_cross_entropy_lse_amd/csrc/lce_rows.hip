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
//   row_state:    0 ignored, 1 valid, 2 label out of range
//   row_key:      label for valid rows, INT_MAX otherwise (sort key)
//   target:       softcapped target logit (valid rows), else 0
//   target_deriv: 1 − tanh²(t_raw / c) at the target (1 without softcap)
//   blocks:       per-block counts of non-ignored and bad rows
// ---------------------------------------------------------------------------
constexpr int kRowsPerPrepBlock = 4;

__global__ void __launch_bounds__(256)
row_prep_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                const int64_t* __restrict__ labels, int64_t N, int64_t H, int64_t V,
                int64_t ignore_index, float softcap, int32_t* __restrict__ row_state,
                int32_t* __restrict__ row_key, float* __restrict__ target,
                float* __restrict__ target_deriv, BlockStats* __restrict__ blocks) {
  __shared__ int counts[kRowsPerPrepBlock][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerPrepBlock + wave;
  int st = kRowIgnored;
  if (row < N) {
    const int64_t y = labels[row];
    st = (y == ignore_index) ? kRowIgnored : ((y >= 0 && y < V) ? kRowValid : kRowBad);
    float t = 0.0f, d = 1.0f;
    if (st == kRowValid) {
      const uint16_t* xr = X + row * H;
      const uint16_t* wr = W + y * H;
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
      dot = wave_sum(dot);
      if (softcap > 0.0f) {
        const float th = tanhf(dot / softcap);
        t = softcap * th;
        d = 1.0f - th * th;
      } else {
        t = dot;
      }
    }
    if (lane == 0) {
      row_state[row] = st;
      if (row_key) row_key[row] = (st == kRowValid) ? (int32_t)y : INT_MAX;
      if (target) target[row] = t;
      if (target_deriv) target_deriv[row] = d;
    }
  }
  if (lane == 0) {
    counts[wave][0] = (st != kRowIgnored);
    counts[wave][1] = (st == kRowBad);
  }
  __syncthreads();
  if (threadIdx.x == 0 && blocks) {
    int nv = 0, nb = 0;
    for (int w = 0; w < kRowsPerPrepBlock; ++w) { nv += counts[w][0]; nb += counts[w][1]; }
    blocks[blockIdx.x] = BlockStats{0.0, nv, nb};
  }
}

int row_prep_blocks(int64_t N) { return (int)((N + kRowsPerPrepBlock - 1) / kRowsPerPrepBlock); }

hipError_t launch_row_prep(const uint16_t* X, const uint16_t* W, const int64_t* labels,
                           int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                           float softcap, int32_t* row_state, int32_t* row_key,
                           float* target, float* target_deriv, BlockStats* blocks,
                           hipStream_t stream) {
  hipLaunchKernelGGL(row_prep_kernel, dim3(row_prep_blocks(N)), dim3(256), 0, stream, X, W,
                     labels, N, H, V, ignore_index, softcap, row_state, row_key, target,
                     target_deriv, blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Merge the S forward partials of each row in split order, then loss and the
// per-block loss sums (fixed-shape tree in double precision).
// ---------------------------------------------------------------------------
constexpr int kFinThreads = 256;

__global__ void __launch_bounds__(kFinThreads)
lse_finalize_kernel(const float* __restrict__ part_m, const float* __restrict__ part_s, int S,
                    int64_t N, const int32_t* __restrict__ row_state,
                    const float* __restrict__ target, float* __restrict__ lse_out,
                    float* __restrict__ loss_out, BlockStats* __restrict__ blocks) {
  __shared__ double ssum[kFinThreads];
  __shared__ int scnt[kFinThreads][2];
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * kFinThreads + tid;
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
    const int st = row_state[row];
    float l = 0.0f;
    if (st == kRowValid) l = lse - target[row];
    else if (st == kRowBad) l = __builtin_nanf("");
    lse_out[row] = lse;
    loss_out[row] = l;
    lossv = (double)l;
    nv = st != kRowIgnored;
    nb = st == kRowBad;
  }
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
  if (tid == 0) blocks[blockIdx.x] = BlockStats{ssum[0], scnt[0][0], scnt[0][1]};
}

int lse_finalize_blocks(int64_t N) { return (int)((N + kFinThreads - 1) / kFinThreads); }

hipError_t launch_lse_finalize(const float* part_m, const float* part_s, int S, int64_t N,
                               const int32_t* row_state, const float* target, float* lse,
                               float* loss, BlockStats* blocks, hipStream_t stream) {
  hipLaunchKernelGGL(lse_finalize_kernel, dim3(lse_finalize_blocks(N)), dim3(kFinThreads), 0,
                     stream, part_m, part_s, S, N, row_state, target, lse, loss, blocks);
  return hipGetLastError();
}

// Fixed-order reduction of the block statistics by one workgroup.
__device__ void reduce_blocks(const BlockStats* __restrict__ blocks, int nblocks, double& sum,
                              int& nv, int& nb) {
  __shared__ double ssum[256];
  __shared__ int scnt[256][2];
  const int tid = threadIdx.x;
  double a = 0.0;
  int v = 0, b = 0;
  for (int i = tid; i < nblocks; i += 256) {
    a += blocks[i].loss_sum;
    v += blocks[i].n_valid;
    b += blocks[i].n_bad;
  }
  ssum[tid] = a;
  scnt[tid][0] = v;
  scnt[tid][1] = b;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      ssum[tid] += ssum[tid + o];
      scnt[tid][0] += scnt[tid + o][0];
      scnt[tid][1] += scnt[tid + o][1];
    }
    __syncthreads();
  }
  sum = ssum[0];
  nv = scnt[0][0];
  nb = scnt[0][1];
}

__global__ void __launch_bounds__(256)
mean_finalize_kernel(const BlockStats* __restrict__ blocks, int nblocks, float* mean,
                     int32_t* n_valid, int32_t* bad_flag) {
  double sum;
  int nv, nb;
  reduce_blocks(blocks, nblocks, sum, nv, nb);
  if (threadIdx.x == 0) {
    *mean = nv > 0 ? (float)(sum / (double)nv) : 0.0f;
    *n_valid = nv;
    if (bad_flag) *bad_flag = nb > 0 ? 1 : 0;
  }
}

hipError_t launch_mean_finalize(const BlockStats* blocks, int nblocks, float* mean,
                                int32_t* n_valid, int32_t* bad_flag, hipStream_t stream) {
  hipLaunchKernelGGL(mean_finalize_kernel, dim3(1), dim3(256), 0, stream, blocks, nblocks, mean,
                     n_valid, bad_flag);
  return hipGetLastError();
}

// scale = dloss / n_valid (0 when no row has a target); counts[0] = n_valid,
// counts[1] = valid rows with an in-range label (the rows that get sorted).
__global__ void __launch_bounds__(256)
scale_finalize_kernel(const BlockStats* __restrict__ blocks, int nblocks,
                      const float* __restrict__ dloss, float* scale, int32_t* counts) {
  double sum;
  int nv, nb;
  reduce_blocks(blocks, nblocks, sum, nv, nb);
  if (threadIdx.x == 0) {
    *scale = nv > 0 ? __fdiv_rn(*dloss, (float)nv) : 0.0f;
    counts[0] = nv;
    counts[1] = nv - nb;
  }
}

hipError_t launch_scale_finalize(const BlockStats* blocks, int nblocks, const float* dloss,
                                 float* scale, int32_t* n_valid, hipStream_t stream) {
  hipLaunchKernelGGL(scale_finalize_kernel, dim3(1), dim3(256), 0, stream, blocks, nblocks,
                     dloss, scale, n_valid);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stable order of the valid rows by label: the position of row i is the number
// of valid rows j with (y_j, j) < (y_i, i).  Quadratic in N but trivially
// parallel and exact; 64 rows per block, each wave scans a quarter of the keys.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
sort_by_label_kernel(const int32_t* __restrict__ row_key, int64_t N, int32_t* __restrict__ sorted) {
  __shared__ int32_t part[4][64];
  const int r = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 64 + r;
  const int32_t ki = row < N ? row_key[row] : INT_MAX;
  const int64_t jb = N * q / 4, je = N * (q + 1) / 4;
  int32_t cnt = 0;
  for (int64_t j = jb; j < je; ++j) {
    const int32_t kj = row_key[j];
    cnt += (kj < ki) | ((kj == ki) & (j < row));
  }
  part[q][r] = cnt;
  __syncthreads();
  if (q == 0 && row < N && ki != INT_MAX) {
    const int32_t pos = part[0][r] + part[1][r] + part[2][r] + part[3][r];
    sorted[pos] = (int32_t)row;
  }
}

hipError_t launch_sort_by_label(const int32_t* row_key, int64_t N, int32_t* sorted,
                                hipStream_t stream) {
  const int grid = (int)((N + 63) / 64);
  hipLaunchKernelGGL(sort_by_label_kernel, dim3(grid), dim3(256), 0, stream, row_key, N, sorted);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dX_i = s · (dX_acc[i] − e_i · w_{y_i})   (valid rows)
//      = 0 (ignored rows), NaN (bad rows)
// The one-hot part −1 · e_i at the target is applied here exactly in fp32.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
dx_finalize_kernel(const float* __restrict__ dX_acc, int64_t N, int64_t H,
                   const int32_t* __restrict__ row_state, const int32_t* __restrict__ row_key,
                   const float* __restrict__ target_deriv, const uint16_t* __restrict__ W,
                   const float* __restrict__ scale, void* __restrict__ dX, int dX_bf16) {
  const int64_t row = blockIdx.x;
  const int st = row_state[row];
  const float s = *scale;
  const float e = target_deriv[row];
  const int64_t y = (st == kRowValid) ? row_key[row] : 0;
  for (int64_t h = (int64_t)threadIdx.x * 4; h < H; h += 1024) {
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (st == kRowValid) {
      const float4 v = *reinterpret_cast<const float4*>(dX_acc + row * H + h);
      const float a[4] = {v.x, v.y, v.z, v.w};
      const u32x2 wv = *reinterpret_cast<const u32x2*>(W + y * H + h);
      const float w4[4] = {__uint_as_float(wv[0] << 16), __uint_as_float(wv[0] & 0xffff0000u),
                           __uint_as_float(wv[1] << 16), __uint_as_float(wv[1] & 0xffff0000u)};
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = s * (a[q] - e * w4[q]);
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

hipError_t launch_dx_finalize(const float* dX_acc, int64_t N, int64_t H,
                              const int32_t* row_state, const int32_t* row_key,
                              const float* target_deriv, const uint16_t* W,
                              const float* scale, void* dX, int dX_bf16, hipStream_t stream) {
  hipLaunchKernelGGL(dx_finalize_kernel, dim3((unsigned)N), dim3(256), 0, stream, dX_acc, N, H,
                     row_state, row_key, target_deriv, W, scale, dX, dX_bf16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dW_v −= s · Σ_{i : y_i = v} e_i · x_i for every label v in [v_lo, v_hi),
// summed over the label's rows in row order (waves take every 4th row, the
// four wave sums are added in wave order).  dst row v − v_lo.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
dw_correct_kernel(const int32_t* __restrict__ sorted, const int32_t* __restrict__ row_key,
                  const int32_t* __restrict__ counts, const float* __restrict__ target_deriv,
                  const uint16_t* __restrict__ X, int64_t H, const float* __restrict__ scale,
                  float* __restrict__ dst, int64_t v_lo, int64_t v_hi) {
  __shared__ float part[4][512];
  const int64_t p = blockIdx.x;
  const int n_ok = counts[1];
  if (p >= n_ok) return;
  const int32_t v = row_key[sorted[p]];
  if (v < v_lo || v >= v_hi) return;
  if (p > 0 && row_key[sorted[p - 1]] == v) return;  // not the start of v's rows
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float s = *scale;
  for (int64_t hc = 0; hc < H; hc += 512) {
    const int64_t h = hc + lane * 8;
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t q = p + wave; q < n_ok; q += 4) {
      const int32_t r = sorted[q];
      if (row_key[r] != v) break;
      if (h < H) {
        const float e = target_deriv[r];
        const u32x4 xv = *reinterpret_cast<const u32x4*>(X + (int64_t)r * H + h);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          a[2 * k] = fmaf(e, __uint_as_float(xv[k] << 16), a[2 * k]);
          a[2 * k + 1] = fmaf(e, __uint_as_float(xv[k] & 0xffff0000u), a[2 * k + 1]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) part[wave][lane * 8 + k] = a[k];
    __syncthreads();
    if (wave == 0 && h < H) {
      float* d = dst + (int64_t)(v - v_lo) * H + h;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float tot = ((part[0][lane * 8 + k] + part[1][lane * 8 + k]) + part[2][lane * 8 + k]) +
                          part[3][lane * 8 + k];
        d[k] -= s * tot;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_dw_correct(const int32_t* sorted, const int32_t* row_key,
                             const int32_t* counts, const float* target_deriv,
                             const uint16_t* X, int64_t N, int64_t H, const float* scale,
                             float* dst, int64_t v_lo, int64_t v_hi, hipStream_t stream) {
  hipLaunchKernelGGL(dw_correct_kernel, dim3((unsigned)N), dim3(256), 0, stream, sorted, row_key,
                     counts, target_deriv, X, H, scale, dst, v_lo, v_hi);
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
