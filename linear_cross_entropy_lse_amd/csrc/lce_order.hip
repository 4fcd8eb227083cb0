// Vocabulary order for the gradient filter, and the row moves of the backward
// on a reordered vocabulary.
//
// The blog "最贵的一层：深入浅出 Liger Kernel 与 Cut Cross-Entropy" (§三) pairs
// CCE's gradient filter with a vocabulary sort: every entry's average logit
// is recorded, and the backward places the entries that are often large next
// to each other, so that whole 256-column blocks fall below the threshold
// more often.
//
// Average logit of entry v over the rows with a target: (1/n)·Σ_i x_i·w_v =
// w_v·x̄ with x̄ the mean of those rows (linearity), so the key costs one
// pass over X (column sums) and one over W (a matrix-vector product, bound
// by HBM: 2·V·H bytes).  Entries are then sorted by decreasing key, equal
// keys by increasing index, through the 64-bit merge sort of the label sort
// (key word: an order-reversing map of the float bits).
//
// The backward on a reordered vocabulary gathers each chunk's W rows into
// position order, runs the unchanged chunk kernels on that copy, and returns
// each dW row to its entry.
#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

namespace {

// Column sums of X over the rows whose label is not ignore_index, one block
// of kMeanRows rows per blockIdx.x, 8 columns per thread; the row count of the
// block goes to cnt[blockIdx.x].  Every sum runs in row order.
__global__ void __launch_bounds__(256)
xsum_partial_kernel(const uint16_t* __restrict__ X, const int64_t* __restrict__ labels,
                    int64_t N, int64_t H, int64_t ignore_index, float* __restrict__ part,
                    int32_t* __restrict__ cnt) {
  const int64_t rb = blockIdx.x;
  const int64_t r0 = rb * kMeanRows;
  const int64_t r1 = r0 + kMeanRows < N ? r0 + kMeanRows : N;
  const int64_t h = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 8;
  const bool col_ok = h < H;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int n = 0;
  for (int64_t r = r0; r < r1; ++r) {
    if (labels[r] == ignore_index) continue;   // the same for the whole block
    ++n;
    if (col_ok) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(X + r * H + h);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += __uint_as_float(v[k] << 16);
        acc[2 * k + 1] += __uint_as_float(v[k] & 0xffff0000u);
      }
    }
  }
  if (col_ok) {
#pragma unroll
    for (int k = 0; k < 8; ++k) part[rb * H + h + k] = acc[k];
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) cnt[rb] = n;
}

// x̄[h] = Σ_rb part[rb][h] / Σ_rb cnt[rb], both in block order; 0 when no
// row has a target.
__global__ void __launch_bounds__(256)
xbar_kernel(const float* __restrict__ part, const int32_t* __restrict__ cnt, int64_t nrb,
            int64_t H, float* __restrict__ xbar) {
  const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (h >= H) return;
  int64_t n = 0;
  float s = 0.0f;
  for (int64_t rb = 0; rb < nrb; ++rb) {
    n += cnt[rb];
    s += part[rb * H + h];
  }
  xbar[h] = n > 0 ? s / (float)n : 0.0f;
}

// Map of a float to a 32-bit word whose unsigned order is the reverse of the
// float order: larger values give smaller words.  −0 and +0 give the same
// word.  Numbers map into [0x007fffff, 0xff800000]; every NaN gives 0, so NaN
// keys come first.
__device__ __forceinline__ uint32_t descending_word(float f) {
  if (f != f) return 0u;
  const uint32_t u = f == 0.0f ? 0u : __float_as_uint(f);
  const uint32_t ascending = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~ascending;
}

// key[v] = w_v·x̄ in fp32: one wave per row, 8 columns per lane per step,
// lane partial sums combined by a fixed butterfly.  word[v] is its sort word.
__global__ void __launch_bounds__(256)
vocab_key_kernel(const uint16_t* __restrict__ W, const float* __restrict__ xbar, int64_t V,
                 int64_t H, float* __restrict__ key, uint32_t* __restrict__ word) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t n_waves = ((int64_t)gridDim.x * 256) >> 6;
  for (int64_t v = wave; v < V; v += n_waves) {
    const uint16_t* row = W + v * H;
    float s = 0.0f;
    for (int64_t h = (int64_t)lane * 8; h < H; h += 512) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + h);
      const float4 xa = *reinterpret_cast<const float4*>(xbar + h);
      const float4 xb = *reinterpret_cast<const float4*>(xbar + h + 4);
      s = fmaf(__uint_as_float(w[0] << 16), xa.x, s);
      s = fmaf(__uint_as_float(w[0] & 0xffff0000u), xa.y, s);
      s = fmaf(__uint_as_float(w[1] << 16), xa.z, s);
      s = fmaf(__uint_as_float(w[1] & 0xffff0000u), xa.w, s);
      s = fmaf(__uint_as_float(w[2] << 16), xb.x, s);
      s = fmaf(__uint_as_float(w[2] & 0xffff0000u), xb.y, s);
      s = fmaf(__uint_as_float(w[3] << 16), xb.z, s);
      s = fmaf(__uint_as_float(w[3] & 0xffff0000u), xb.w, s);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) {
      key[v] = s;
      word[v] = descending_word(s);
    }
  }
}

__global__ void __launch_bounds__(256)
order_extract_kernel(const uint64_t* __restrict__ keys, int64_t V, int32_t* __restrict__ order) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < V) order[j] = (int32_t)(uint32_t)keys[j];
}

// pos1[order[j]] = j + 1 for every in-range entry (pos1 cleared before).
__global__ void __launch_bounds__(256)
position_kernel(const int32_t* __restrict__ order, int64_t V, int32_t* __restrict__ pos1) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= V) return;
  const int32_t v = order[j];
  if (v >= 0 && v < V) pos1[v] = (int32_t)(j + 1);
}

// Label key of each row moved to its position; rows without an in-range
// label, or whose label has no position, keep the key INT_MAX.
__global__ void __launch_bounds__(256)
position_keys_kernel(const int32_t* __restrict__ key, int64_t N, int64_t V,
                     const int32_t* __restrict__ pos1, int32_t* __restrict__ pkey) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const int32_t k = key[i];
  const int32_t p = (k >= 0 && k < V) ? pos1[k] : 0;
  pkey[i] = p > 0 ? p - 1 : INT32_MAX;
}

// Wp[j] = W[order[j0 + j]] for j < rows (16-byte moves, one wave per row);
// an out-of-range entry gives a zero row.
__global__ void __launch_bounds__(256)
gather_rows_kernel(const uint16_t* __restrict__ W, int64_t V, int64_t H,
                   const int32_t* __restrict__ order, int64_t j0, int64_t rows,
                   uint16_t* __restrict__ Wp) {
  const int lane = threadIdx.x & 63;
  const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (j >= rows) return;
  const int32_t v = order[j0 + j];
  const bool ok = v >= 0 && v < V;
  const u32x4* src = reinterpret_cast<const u32x4*>(W + (ok ? (int64_t)v : 0) * H);
  u32x4* dst = reinterpret_cast<u32x4*>(Wp + j * H);
  for (int64_t q = lane; q < H / 8; q += 64) dst[q] = ok ? src[q] : u32x4{0u, 0u, 0u, 0u};
}

// dW[order[j0 + j]] = src[j] (fp32 rows) as fp32 or bf16 (nearest even);
// out-of-range entries are skipped.
template <bool kBf16>
__global__ void __launch_bounds__(256)
scatter_rows_kernel(const float* __restrict__ src, int64_t V, int64_t H,
                    const int32_t* __restrict__ order, int64_t j0, int64_t rows,
                    void* __restrict__ dW) {
  const int lane = threadIdx.x & 63;
  const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (j >= rows) return;
  const int32_t v = order[j0 + j];
  if (v < 0 || v >= V) return;
  const float4* s = reinterpret_cast<const float4*>(src + j * H);
  for (int64_t q = lane; q < H / 4; q += 64) {
    const float4 x = s[q];
    if (kBf16) {
      u32x2 pk;
      pk[0] = f32_to_bf16_bits(x.x) | (f32_to_bf16_bits(x.y) << 16);
      pk[1] = f32_to_bf16_bits(x.z) | (f32_to_bf16_bits(x.w) << 16);
      reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dW) + (int64_t)v * H)[q] = pk;
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(dW) + (int64_t)v * H)[q] = x;
    }
  }
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

hipError_t launch_vocab_key(const uint16_t* X, const int64_t* labels, int64_t N, int64_t H,
                            const uint16_t* W, int64_t V, int64_t ignore_index, float* part,
                            int32_t* cnt, float* xbar, float* key, uint32_t* word,
                            hipStream_t stream) {
  const int64_t nrb = mean_row_blocks(N);
  if (nrb > 0)
    hipLaunchKernelGGL(xsum_partial_kernel, dim3((unsigned)nrb, (unsigned)((H / 8 + 255) / 256)),
                       dim3(256), 0, stream, X, labels, N, H, ignore_index, part, cnt);
  hipLaunchKernelGGL(xbar_kernel, dim3(blocks_for(H)), dim3(256), 0, stream, part, cnt, nrb, H,
                     xbar);
  int64_t grid = (V + 3) / 4;   // 4 rows (waves) per block, at most 8 rows per wave
  if (grid > 32768) grid = 32768;
  hipLaunchKernelGGL(vocab_key_kernel, dim3((unsigned)grid), dim3(256), 0, stream, W, xbar, V, H,
                     key, word);
  return hipGetLastError();
}

hipError_t launch_order_extract(const uint64_t* keys, int64_t V, int32_t* order,
                                hipStream_t stream) {
  hipLaunchKernelGGL(order_extract_kernel, dim3(blocks_for(V)), dim3(256), 0, stream, keys, V,
                     order);
  return hipGetLastError();
}

hipError_t launch_position_keys(const int32_t* order, int64_t V, const int32_t* key, int64_t N,
                                int32_t* pos1, int32_t* pkey, hipStream_t stream) {
  hipError_t e = launch_fill_zero(pos1, (V * 4 + 15) / 16 * 16, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(position_kernel, dim3(blocks_for(V)), dim3(256), 0, stream, order, V, pos1);
  hipLaunchKernelGGL(position_keys_kernel, dim3(blocks_for(N)), dim3(256), 0, stream, key, N, V,
                     pos1, pkey);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* W, int64_t V, int64_t H, const int32_t* order,
                              int64_t j0, int64_t rows, uint16_t* Wp, hipStream_t stream) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks_for(rows * 64)), dim3(256), 0, stream, W, V,
                     H, order, j0, rows, Wp);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* src, int64_t V, int64_t H, const int32_t* order,
                               int64_t j0, int64_t rows, void* dW, int bf16, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL(scatter_rows_kernel<true>, dim3(blocks_for(rows * 64)), dim3(256), 0,
                       stream, src, V, H, order, j0, rows, dW);
  else
    hipLaunchKernelGGL(scatter_rows_kernel<false>, dim3(blocks_for(rows * 64)), dim3(256), 0,
                       stream, src, V, H, order, j0, rows, dW);
  return hipGetLastError();
}

}  // namespace lce
