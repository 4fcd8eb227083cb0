// MFMA kernels of liblce for gfx950: the three N·H·V contractions of the
// linear cross-entropy and their fused epilogues.
//
//   lse_partials_kernel   forward: Z tile = W_J · X_Iᵀ, optional softcap, and a
//                         running (max, Σexp) per token kept in registers across
//                         the vocabulary tiles of one split; one (m, s) partial
//                         per token and split is written, never the logits.
//                         (blog "最贵的一层：深入浅出 Liger Kernel 与 Cut
//                         Cross-Entropy", §三: tiles staged on chip, in-tile LSE,
//                         merge m' = max(m, m_b), s' = s·e^(m−m') + s_b·e^(m_b−m');
//                         AI-infra KB M011 §05: first tile initialises)
//   grad_logits_kernel    backward: the same tile product recomputed, p =
//                         exp(z − LSE), times the softcap derivative (Unsloth
//                         fused-CE chapter §4), written as bf16 into a chunk of
//                         the vocabulary (M011 §06: recompute the tile from the
//                         saved LSE)
//   dx_gemm_kernel        dX partial += G_chunk · W_chunk  (M011 §06: dH += dZ·W)
//   dw_gemm_kernel        dW_chunk = s · G_chunkᵀ · X      (M011 §06: dW += dZᵀ·H)
//
// The pages merge per-tile LSEs with spin-locked atomics; here every
// (token tile, split) writes its own partial and a second pass merges them in
// a fixed order, so results are bitwise reproducible.
#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

// One 256x256 tile over K range [k_begin, k_end).  The shared buffer holds two
// pipeline stages of both operands (128 KiB).
template <class LA, class LB>
__device__ __forceinline__ void gemm_tile(const uint16_t* __restrict__ A, int64_t lda,
                                          int64_t a_row0, int64_t a_rows, int64_t a_ktotal,
                                          const uint16_t* __restrict__ B, int64_t ldb,
                                          int64_t b_row0, int64_t b_rows, int64_t b_ktotal,
                                          int64_t k_begin, int64_t k_end, uint16_t* smem,
                                          f32x16 (&acc)[kMI][kNI]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t nsteps = (k_end - k_begin + kBK - 1) / kBK;
  if (nsteps <= 0) return;
  uint16_t* sA[2] = {smem, smem + kStageElems};
  uint16_t* sB[2] = {smem + 2 * kStageElems, smem + 3 * kStageElems};
  LA la;
  LB lb;
  la.init(A, lda, a_row0, a_rows, a_ktotal, tid);
  lb.init(B, ldb, b_row0, b_rows, b_ktotal, tid);
  la.load(k_begin);
  lb.load(k_begin);
  __syncthreads();  // the previous tile's last readers of stage 0 are done
  la.store(sA[0], tid);
  lb.store(sB[0], tid);
  __syncthreads();
  for (int64_t step = 0; step < nsteps; ++step) {
    const int cur = (int)(step & 1);
    const bool more = step + 1 < nsteps;
    if (more) {
      const int64_t k = k_begin + (step + 1) * kBK;
      la.load(k);
      lb.load(k);
    }
    mfma_step(sA[cur], sB[cur], wm, wn, lane, acc);
    if (more) {
      la.store(sA[cur ^ 1], tid);
      lb.store(sB[cur ^ 1], tid);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Forward: per (token tile, vocabulary split) partial (max, sum-exp).
// Values are kept in base 2: u = z·log2(e), s = Σ 2^(u − m).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads, 1)
lse_partials_kernel(LseParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kStageElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int ti = g % p.T, split = g / p.T;
  const int j0 = (int)((int64_t)split * p.n_vtiles / p.S);
  const int j1 = (int)((int64_t)(split + 1) * p.n_vtiles / p.S);
  const int64_t tok0 = (int64_t)ti * kTile;
  const bool capped = p.softcap > 0.0f;
  const float k2 = capped ? 2.0f * kLog2e / p.softcap : 0.0f;
  const float c2 = capped ? p.softcap * kLog2e : kLog2e;
  const float NEG_INF = -__builtin_inff();

  float m[kNI], s[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) { m[ni] = NEG_INF; s[ni] = 0.0f; }

  f32x16 acc[kMI][kNI];
  for (int j = j0; j < j1; ++j) {
    const int64_t v0 = (int64_t)j * kTile;
    zero_acc(acc);
    gemm_tile<KMajorTile, KMajorTile>(p.W, p.H, v0, p.V, p.H, p.X, p.H, tok0, p.N, p.H, 0, p.H,
                                      smem, acc);
    // Vocabulary rows of this tile at or beyond V are masked: row_const >= lim.
    const int lim = (int)(p.V - v0 < kTile ? p.V - v0 : kTile) - acc_row_lane(wm, lane);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      float tmax = NEG_INF;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float z = acc[mi][ni][r];
          float u = capped ? c2 * tanh_of_scaled(z, k2) : z * kLog2e;
          if (acc_row_const(mi, r) >= lim) u = NEG_INF;
          acc[mi][ni][r] = u;
          tmax = fmaxf(tmax, u);
        }
      const float mn = fmaxf(m[ni], tmax);
      if (mn == NEG_INF) continue;  // no valid vocabulary row seen yet
      float sum = 0.0f;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += exp2_fast(acc[mi][ni][r] - mn);
      s[ni] = s[ni] * exp2_fast(m[ni] - mn) + sum;
      m[ni] = mn;
    }
  }

  // Lanes l and l^32 hold the same token column (different vocabulary rows).
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const float m2 = __shfl_xor(m[ni], 32);
    const float s2 = __shfl_xor(s[ni], 32);
    const float mn = fmaxf(m[ni], m2);
    if (mn != NEG_INF) {
      s[ni] = s[ni] * exp2_fast(m[ni] - mn) + s2 * exp2_fast(m2 - mn);
      m[ni] = mn;
    }
  }
  // Waves wm = 0 and wm = 1 cover the two vocabulary halves of the same tokens.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int col = acc_col(wn, ni, lane);
      red[col] = m[ni];
      red[kTile + col] = s[ni];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int col = acc_col(wn, ni, lane);
      const float m2 = red[col], s2 = red[kTile + col];
      float mm = m[ni], ss = s[ni];
      const float mn = fmaxf(mm, m2);
      if (mn != NEG_INF) {
        ss = ss * exp2_fast(mm - mn) + s2 * exp2_fast(m2 - mn);
        mm = mn;
      }
      const int64_t tok = tok0 + col;
      if (tok < p.N) {
        p.part_m[(int64_t)split * p.N + tok] = mm;
        p.part_s[(int64_t)split * p.N + tok] = ss;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, step 1: recompute the logits of one vocabulary chunk and write
// G = p · (1 − tanh²) (the dense part of dZ before the 1/n_valid scale) as
// bf16 into G[token][v − v_begin].  Ignored rows give 0, bad rows NaN,
// vocabulary rows beyond V give 0.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads, 1)
grad_logits_kernel(GradParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kStageElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int ti = g % p.T, split = g / p.T;
  const int j0 = (int)((int64_t)split * p.n_vtiles / p.S);
  const int j1 = (int)((int64_t)(split + 1) * p.n_vtiles / p.S);
  const int64_t tok0 = (int64_t)ti * kTile;
  const bool capped = p.softcap > 0.0f;
  const float k2 = capped ? 2.0f * kLog2e / p.softcap : 0.0f;
  const float c2 = capped ? p.softcap * kLog2e : kLog2e;
  const float qnan = __builtin_nanf("");

  // Per token column: base-2 LSE and the row class (fixed for all tiles).
  float lse2[kNI], rscale[kNI];
  bool tok_ok[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t tok = tok0 + acc_col(wn, ni, lane);
    tok_ok[ni] = tok < p.N;
    const int st = tok_ok[ni] ? p.row_state[tok] : (int)kRowIgnored;
    lse2[ni] = tok_ok[ni] ? p.lse[tok] * kLog2e : 0.0f;
    rscale[ni] = st == kRowValid ? 1.0f : (st == kRowBad ? qnan : 0.0f);
  }

  f32x16 acc[kMI][kNI];
  for (int j = j0; j < j1; ++j) {
    const int64_t vloc0 = (int64_t)j * kTile;      // chunk-local vocabulary row
    const int64_t v0 = p.v_begin + vloc0;          // global vocabulary row
    zero_acc(acc);
    gemm_tile<KMajorTile, KMajorTile>(p.W, p.H, v0, p.V, p.H, p.X, p.H, tok0, p.N, p.H, 0, p.H,
                                      smem, acc);
    const int lim = (int)(p.V - v0 < kTile ? p.V - v0 : kTile) - acc_row_lane(wm, lane);
    const int64_t vl_lane = vloc0 + acc_row_lane(wm, lane);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      uint16_t* grow = p.G + (tok0 + acc_col(wn, ni, lane)) * p.ldg + vl_lane;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float gv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = gq * 4 + q;
            const float z = acc[mi][ni][r];
            float u, d;
            if (capped) {
              const float t = tanh_of_scaled(z, k2);
              u = c2 * t;
              d = 1.0f - t * t;
            } else {
              u = z * kLog2e;
              d = 1.0f;
            }
            float val = exp2_fast(u - lse2[ni]) * d * rscale[ni];
            if (acc_row_const(mi, r) >= lim) val = 0.0f;
            gv[q] = val;
          }
          if (tok_ok[ni]) {
            u32x2 packed;
            packed[0] = f32_to_bf16_bits(gv[0]) | (f32_to_bf16_bits(gv[1]) << 16);
            packed[1] = f32_to_bf16_bits(gv[2]) | (f32_to_bf16_bits(gv[3]) << 16);
            *reinterpret_cast<u32x2*>(grow + acc_row_const(mi, gq * 4)) = packed;
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward, step 2: dXp[split] (+)= G[:, k-range] · W[v_begin + k-range, :].
// M = tokens (A = G, K-major), N = hidden (B = W chunk, stored [K, N]).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads, 1)
dx_gemm_kernel(DxParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kStageElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = p.nt_tok * p.nt_h;
  const int split = g / per_split;
  const int g2 = g % per_split;
  const int64_t tok0 = (int64_t)(g2 / p.nt_h) * kTile;
  const int64_t h0 = (int64_t)(g2 % p.nt_h) * kTile;
  const int64_t steps = (p.k_len + kBK - 1) / kBK;
  const int64_t k_begin = (steps * split / p.KS) * kBK;
  const int64_t k_end = (steps * (split + 1) / p.KS) * kBK;

  f32x16 acc[kMI][kNI];
  zero_acc(acc);
  gemm_tile<KMajorTile, MNMajorTile>(p.G, p.ldg, tok0, p.N, p.ldg,
                                     p.Wc, p.H, h0, p.H, p.wc_rows,
                                     k_begin, k_end, smem, acc);
  float* dst = p.dXp + (int64_t)split * p.N * p.H;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int64_t h = h0 + acc_col(wn, ni, lane);
      if (h >= p.H) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t tok = tok0 + acc_row(wm, mi, r, lane);
        if (tok < p.N) {
          float* q = dst + tok * p.H + h;
          *q = p.accumulate ? *q + acc[mi][ni][r] : acc[mi][ni][r];
        }
      }
    }
}

// ---------------------------------------------------------------------------
// Backward, step 3: dst[v_local][h] = s · Σ_tok G[tok][v_local] · X[tok][h].
// M = chunk vocabulary (A = G, stored [K, M]), N = hidden (B = X, [K, N]).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads, 1)
dw_gemm_kernel(DwParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * kStageElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t vt0 = (int64_t)(g / p.nt_h) * kTile;
  const int64_t h0 = (int64_t)(g % p.nt_h) * kTile;

  f32x16 acc[kMI][kNI];
  zero_acc(acc);
  gemm_tile<MNMajorTile, MNMajorTile>(p.G, p.ldg, vt0, p.ldg, p.N,
                                      p.X, p.H, h0, p.H, p.N,
                                      0, p.N, smem, acc);
  const float sc = *p.scale;
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int64_t h = h0 + acc_col(wn, ni, lane);
      if (h >= p.H) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t vl = vt0 + acc_row(wm, mi, r, lane);
        if (vl < p.chunk_len) p.dst[vl * p.H + h] = sc * acc[mi][ni][r];
      }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_lse_partials(const LseParams& p, hipStream_t stream) {
  const int grid = p.T * p.S;
  hipLaunchKernelGGL(lse_partials_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_grad_logits(const GradParams& p, hipStream_t stream) {
  const int grid = p.T * p.S;
  hipLaunchKernelGGL(grad_logits_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dx_gemm(const DxParams& p, hipStream_t stream) {
  const int grid = p.nt_tok * p.nt_h * p.KS;
  hipLaunchKernelGGL(dx_gemm_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_dw_gemm(const DwParams& p, hipStream_t stream) {
  const int grid = p.nt_v * p.nt_h;
  hipLaunchKernelGGL(dw_gemm_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lce
