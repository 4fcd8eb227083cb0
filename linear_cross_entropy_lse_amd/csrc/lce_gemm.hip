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
//   chunk_gemm_kernel     per vocabulary chunk, one launch holding both
//                         dX_acc += G_chunk · W_chunk       (M011 §06: dH += dZ·W)
//                         dW_chunk = s · G_chunkᵀ · X       (M011 §06: dW += dZᵀ·H)
//
// The pages merge per-tile LSEs with spin-locked atomics; here every
// (token tile, split) writes its own partial and a second pass merges them in
// a fixed order, so results are bitwise reproducible.
#include "lce_device.h"
#include "lce_internal.h"

namespace lce {

// ---------------------------------------------------------------------------
// Forward: per (token tile, vocabulary split) partial (max, sum-exp).
// Values are kept in base 2: u = z·log2(e), s = Σ 2^(u − m).
//
// Epilogue modes (kMode):
//   kPlain     no softcap: a max pass over the tile's raw logits, then the
//              sum pass against the merged running max.
//   kCapFixed  softcap c with 2c·log2(e) < 120: u = c·log2(e)·tanh(z/c) is
//              bounded by c2 = c·log2(e), so the fixed reference m = c2 needs
//              no max pass; every term 2^(u − c2) lies in [2^(−2·c2), 1],
//              above the smallest normal float.  With r = 1/(2^(z·k2) + 1),
//              u − c2 = −2·c2·r.
//   kCapGeneral softcap too large for the fixed reference: max pass on raw z
//              (tanh is increasing), then the sum pass.
// ---------------------------------------------------------------------------
enum EpiMode { kPlain = 0, kCapFixed = 1, kCapGeneral = 2 };

// Fold one finished 256 x 256 logit tile into the per-column running (m, s).
// kMasked: vocabulary rows at or beyond V are present in this tile (only the
// last one); row_const >= lim marks them.  Split out so that every other tile
// runs without per-element tests.  The logit scale a is folded into k2 and
// l2a = a·log2(e).  kZSum (label smoothing): zs gathers the per-column sum of
// the final logits in units of the softcap (capped modes: Σ tanh) or of the
// raw product (plain mode: Σ z); the caller rescales it.
template <int kMode, bool kMasked, bool kZSum>
__device__ __forceinline__ void lse_fold_tile(const f32x16 (&acc)[kMI][kNI], float (&m)[kNI],
                                              float (&s)[kNI], float (&zs)[kNI], int lim, float k2,
                                              float c2, float l2a) {
  const float NEG_INF = -__builtin_inff();
  const float inv2c2 = kMode == kCapFixed ? 0.5f / c2 : 0.0f;
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    float mref = m[ni];
    if (kMode != kCapFixed) {
      float zmax = NEG_INF;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float z = acc[mi][ni][r];
          zmax = fmaxf(zmax, (!kMasked || acc_row_const(mi, r) < lim) ? z : NEG_INF);
        }
      const float umax = kMode == kPlain ? zmax * l2a
                                         : (zmax == NEG_INF ? NEG_INF : c2 * tanh_of_scaled(zmax, k2));
      const float mn = fmaxf(m[ni], umax);
      mref = mn == NEG_INF ? 0.0f : mn;   // nothing valid yet: every term is an exact 0
      s[ni] *= exp2_fast(m[ni] - mref);
      m[ni] = mn;
    }
    float sum = 0.0f, zsum = 0.0f;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float z = acc[mi][ni][r];
        const bool ok = !kMasked || acc_row_const(mi, r) < lim;
        float e, zt = 0.0f;
        if (kMode == kPlain) {
          e = exp2_fast(fmaf(z, l2a, -mref));
          zt = z;
        } else if (kMode == kCapFixed) {
          // q = 2c2·r, as the reciprocal of (2^(z·k2) + 1)/(2c2): e = 2^(−q)
          const float q = rcp_fast(fmaf(exp2_fast(z * k2), inv2c2, inv2c2));
          e = exp2_fast(-q);
          zt = fmaf(-2.0f * inv2c2, q, 1.0f);   // tanh = 1 − 2r = 1 − q/c2
        } else {
          const float t = tanh_of_scaled(z, k2);
          e = exp2_fast(c2 * t - mref);
          zt = t;
        }
        sum += ok ? e : 0.0f;
        if (kZSum) zsum += ok ? zt : 0.0f;
      }
    s[ni] += sum;
    if (kZSum) zs[ni] += zsum;
  }
}

// End of a (token tile, split) sweep: merge the running (m, s) (and Σ z) of
// the lane pairs and of the two vocabulary halves, then write one partial
// per token of the split.  `red` is LDS scratch of 3·256 floats; the caller
// has drained every load into LDS.
template <int kMode, bool kZSum>
__device__ __forceinline__ void store_split_partials(float (&m)[kNI], float (&s)[kNI],
                                                     float (&zs)[kNI], float* red, int wm, int wn,
                                                     int lane, int64_t tok0, int split, int64_t N,
                                                     int64_t ldp, float zunit, float* part_m,
                                                     float* part_s, float* part_z) {
  const float NEG_INF = -__builtin_inff();
  // Lanes l and l^32 hold the same token column (different vocabulary rows).
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const float m2 = __shfl_xor(m[ni], 32);
    const float s2 = __shfl_xor(s[ni], 32);
    const float mn = fmaxf(m[ni], m2);
    const float mref = mn == NEG_INF ? 0.0f : mn;
    s[ni] = s[ni] * exp2_fast(m[ni] - mref) + s2 * exp2_fast(m2 - mref);
    m[ni] = mn;
    if (kZSum) zs[ni] += __shfl_xor(zs[ni], 32);
  }
  // Waves wm = 0 and wm = 1 cover the two vocabulary halves of the same tokens.
  __syncthreads();
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int col = acc_col(wn, ni, lane);
      red[col] = m[ni];
      red[kTile + col] = s[ni];
      if (kZSum) red[2 * kTile + col] = zs[ni];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int col = acc_col(wn, ni, lane);
      const float m2 = red[col], s2 = red[kTile + col];
      const float mn = fmaxf(m[ni], m2);
      const float mref = mn == NEG_INF ? 0.0f : mn;
      const float ss = s[ni] * exp2_fast(m[ni] - mref) + s2 * exp2_fast(m2 - mref);
      const int64_t tok = tok0 + col;
      if (tok < N) {
        part_m[(int64_t)split * ldp + tok] = mn;
        part_s[(int64_t)split * ldp + tok] = ss;
        // Σ z in natural units: c·Σ tanh (capped) or a·Σ (x·w) (plain).
        if (kZSum) part_z[(int64_t)split * ldp + tok] = zunit * (zs[ni] + red[2 * kTile + col]);
      }
    }
  }
}

template <bool kTail, int kMode, bool kZSum>
__global__ void __launch_bounds__(kThreads, 1)
lse_partials_kernel(LseParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[4 * kStageElems];
  LCE_LDS uint16_t* smem = (LCE_LDS uint16_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  int ti, split;
  grid_tile(g, p.T, p.tt, p.ss, ti, split);
  const int j0 = (int)((int64_t)split * p.n_vtiles / p.S);
  const int j1 = (int)((int64_t)(split + 1) * p.n_vtiles / p.S);
  const int64_t tok0 = (int64_t)ti * kTile;
  const float k2 = kMode != kPlain ? 2.0f * kLog2e * p.logit_scale / p.softcap : 0.0f;
  const float c2 = kMode != kPlain ? p.softcap * kLog2e : 0.0f;
  const float l2a = kLog2e * p.logit_scale;
  const float NEG_INF = -__builtin_inff();

  float m[kNI], s[kNI], zs[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    m[ni] = kMode == kCapFixed ? c2 : NEG_INF;
    s[ni] = 0.0f;
    zs[ni] = 0.0f;
  }

  // Tiles j < j_mid have every vocabulary row below V; the one tile that
  // reaches past V (if this split holds it) runs in a loop of its own with the
  // masked fold, so the common path carries no per-element tests.
  const int j_mid = (int)(j1 < p.V / kTile ? j1 : (j0 > p.V / kTile ? j0 : p.V / kTile));
  // Every tile prefetches the first two steps of the next one (same token
  // tile, next vocabulary rows) while its fold runs.
  Sweep sw;
  f32x16 acc[kMI][kNI];
  for (int j = j0; j < j_mid; ++j) {
    gemm_tile<false, false, kTail, true>(p.W, p.H, (int64_t)j * kTile, p.V, p.X, p.H, tok0, p.N, 0,
                                         p.H, p.H, smem, acc, &sw,
                                         j + 1 < j1 ? (int64_t)(j + 1) * kTile : -1);
    lse_fold_tile<kMode, false, kZSum>(acc, m, s, zs, 0, k2, c2, l2a);
  }
  for (int j = j_mid; j < j1; ++j) {
    const int64_t v0 = (int64_t)j * kTile;
    gemm_tile<false, false, kTail, true>(p.W, p.H, v0, p.V, p.X, p.H, tok0, p.N, 0, p.H, p.H, smem,
                                         acc, &sw, j + 1 < j1 ? v0 + kTile : -1);
    const int lim = (int)(p.V - v0) - acc_row_lane(wm, lane);
    lse_fold_tile<kMode, true, kZSum>(acc, m, s, zs, lim, k2, c2, l2a);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   // the last tile's (empty) prefetch has landed
  store_split_partials<kMode, kZSum>(m, s, zs, reinterpret_cast<float*>(smem_raw), wm, wn, lane,
                                     tok0, split, p.N, p.ldp,
                                     kMode == kPlain ? p.logit_scale : p.softcap, p.part_m,
                                     p.part_s, p.part_z);
}

// ---------------------------------------------------------------------------
// Backward, step 1: recompute the logits of one vocabulary chunk and write
// G = p · (1 − tanh²) (the dense part of dZ before the 1/n_valid scale) as
// bf16 into G[token][v − v_begin].  Ignored rows give 0, bad rows NaN,
// vocabulary rows beyond V give 0.  With softcap, r = 1/(2^(z·k2) + 1) gives
// tanh = 1 − 2r, p = 2^((c2 − lse2) − 2·c2·r) and 1 − tanh² = 4r(1 − r).
//
// The kernel also looks for an entry whose softmax exceeds 1/2 + 2^-10 (at
// most one per row): a max over each lane's softmax values of a token column
// against 1/2, and, for the rare tile that holds one, the W row of the lane's
// first row of the tile goes to GradParams::dom_base.  The exact entries
// themselves are computed afterwards (launch_exact_entries).
// ---------------------------------------------------------------------------
// G of one finished tile, as bf16, through the G descriptor (rows past N are
// out of range).  Plain form (kGen false): G = p·d, off[ni] folding the row
// class in (−inf for ignored rows, so G = 0; NaN for rows with a bad label).
// General form: G = gsc[ni]·(c1[ni]·p − eps_v)·d with the row's scale gsc (0
// ignored, NaN bad) and Z-loss factor c1.  kMasked: the tile reaches past V
// and rows with row_const >= lim are written as 0.
// kFilter: also report whether any value of the dense part compared by the
// gradient filter, (1 + 2l·LSE)·p over rows with a target, is not below
// `feps` (NaN counts as not below).
// Stores follow the blocked G layout.  A lane holds rows 4·(lane/32) + 0..3 of
// each 8-row group gq of its mi block; lanes l and l + 32 trade halves
// (permlane32 swap) so that lane l stores the 8 rows of group 2gp and lane
// l + 32 those of group 2gp + 1, 16 bytes each: sub-block mi/2, column
// (mi%2)·32 + 16gp (+ 8 from the lane half, carried by cb).
// pmax[ni] gathers the largest softmax value of each token column among the
// lane's rows, times 4 with softcap (for the dominance check,
// grad_mark_candidates).
// kSplit (precise gradient): each value g is stored as hi = bf16(g) through
// rs and lo = bf16(g − hi) through rs_lo, at the same offsets.
template <bool kCapped, bool kMasked, bool kGen, bool kFilter = false, bool kSplit = false>
__device__ __forceinline__ bool grad_store_tile(const f32x16 (&acc)[kMI][kNI], const float (&off)[kNI],
                                                const float (&gsc)[kNI], const float (&c1)[kNI],
                                                float eps_v, __amdgpu_buffer_rsrc_t rs,
                                                __amdgpu_buffer_rsrc_t rs_lo,
                                                const uint32_t (&cb)[kNI], int lim, float k2,
                                                float c2, float l2a, float feps,
                                                float (&pmax)[kNI]) {
  bool active = false;
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        u32x2 pk[2], lo[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gq = 2 * gp + h;
          float gv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = gq * 4 + q;
            const float z = acc[mi][ni][r];
            float val, pr, pm;
            if (kCapped) {
              // off carries + 2 here: pr4 = 4p, and 4p·r(1 − r) = p·(1 − tanh²).
              const float rr = rcp_fast(exp2_fast(z * k2) + 1.0f);
              const float pr4 = exp2_fast(fmaf(-2.0f * c2, rr, off[ni]));
              const float dq = fmaf(-rr, rr, rr);
              val = kGen ? gsc[ni] * fmaf(c1[ni], pr4, -4.0f * eps_v) * dq : pr4 * dq;
              pr = 0.25f * pr4;   // read by the filter only
              pm = pr4;
            } else {
              pr = exp2_fast(fmaf(z, l2a, off[ni]));
              val = kGen ? gsc[ni] * fmaf(c1[ni], pr, -eps_v) : pr;
              pm = pr;
            }
            gv[q] = (!kMasked || acc_row_const(mi, r) < lim) ? val : 0.0f;
            pmax[ni] = fmaxf(pmax[ni], (!kMasked || acc_row_const(mi, r) < lim) ? pm : 0.0f);
            if (kFilter) {
              // Plain form: ignored rows have pr = 0, bad rows NaN.
              const float fv = kGen ? (gsc[ni] != 0.0f ? c1[ni] * pr : 0.0f) : pr;
              active |= (!kMasked || acc_row_const(mi, r) < lim) && !(fv < feps);
            }
          }
          pk[h][0] = pack_bf16x2(gv[0], gv[1]);
          pk[h][1] = pack_bf16x2(gv[2], gv[3]);
          if (kSplit) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
              lo[h][e] = pack_bf16x2(gv[2 * e] - __uint_as_float(pk[h][e] << 16),
                                     gv[2 * e + 1] - __uint_as_float(pk[h][e] & 0xffff0000u));
          }
        }
        const uint32_t eo = (uint32_t)((mi >> 1) * kGSubElems + (mi & 1) * 32 + 16 * gp);
        const auto s0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
        const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
        __builtin_amdgcn_raw_buffer_store_b128(out, rs, (int)(cb[ni] + 2u * eo), 0, 0);
        if (kSplit) {
          const auto t0 = __builtin_amdgcn_permlane32_swap(lo[0][0], lo[1][0], false, false);
          const auto t1 = __builtin_amdgcn_permlane32_swap(lo[0][1], lo[1][1], false, false);
          const u32x4 out_lo = {t0[0], t1[0], t0[1], t1[1]};
          __builtin_amdgcn_raw_buffer_store_b128(out_lo, rs_lo, (int)(cb[ni] + 2u * eo), 0, 0);
        }
      }
  return active;
}

// Filter flag of one wave's quarter of tile (ti, j): byte `wave` of word
// ti·n_vtiles + j, written by lane 0.
__device__ __forceinline__ void store_filter_flag(uint8_t* flags, bool active, int ti, int j,
                                                  int n_vtiles, int wave, int lane) {
  const bool any = __builtin_amdgcn_ballot_w64(active) != 0;
  if (lane == 0) flags[((int64_t)ti * n_vtiles + j) * 4 + wave] = any ? 1 : 0;
}

// Candidates of a dominant entry in one stored tile: for each token column ni
// of this lane, whether its largest softmax value among the lane's rows
// (pmax, from grad_store_tile; 4p with softcap) exceeds 1/2.  That is a
// superset of the entries above 1/2 + 2^-10: the exact-entry kernel
// recomputes the candidate tile's logits and keeps an entry only if its logit
// lies above the row's dominance threshold.  A candidate leaves tile number
// j + 1 in the lane's LDS slot of the column (an LDS max without return, so
// the epilogue neither waits nor branches); grad_store_candidates turns the
// slots into W rows after the sweep.  Rows without a gradient (ignored, bad
// label) have p = 0 or NaN in the plain form and are never candidates; in the
// general form the exact-entry kernel drops them.
template <bool kCapped>
__device__ __forceinline__ void grad_mark_candidates(const float (&pmax)[kNI],
                                                     uint32_t (*cand)[kThreads], int tid, int j) {
  const float thr = kCapped ? 2.0f : 0.5f;
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni)
    atomicMax(&cand[ni][tid], pmax[ni] > thr ? (uint32_t)(j + 1) : 0u);
}

// After the sweep: the W row of the lane's first row of the candidate tile,
// plus key_offset, for the token of each marked column.  The output pointer
// and v_begin + key_offset come from LDS (dom: [0], [1]), and tok0 from the
// token tile ti, so that none of them stays in a register through the sweep.
__device__ __forceinline__ void grad_store_candidates(const uint32_t (*cand)[kThreads],
                                                      const int64_t* dom, int tid, int ti, int wn,
                                                      int lane, int lrow) {
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const uint32_t c = cand[ni][tid];
    if (c != 0u) {
      int32_t* dom_base = reinterpret_cast<int32_t*>(dom[0]);
      dom_base[(int64_t)ti * kTile + acc_col(wn, ni, lane)] =
          (int32_t)(dom[1] + (int64_t)(c - 1u) * kTile + lrow);
    }
  }
}

template <bool kTail, bool kCapped, bool kGen, bool kFilter, bool kSplit = false>
__global__ void __launch_bounds__(kThreads, 1)
grad_logits_kernel(GradParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[4 * kStageElems];
  __shared__ uint32_t s_cand[kNI][kThreads];   // candidate tile + 1 per token column (0: none)
  __shared__ int64_t s_dom[2];                 // dom_base and v_begin + key_offset
  LCE_LDS uint16_t* smem = (LCE_LDS uint16_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int ti, split;
  if (p.round_tiles > 0) {
    round_tile(blockIdx.x, p.round_tiles, ti, split);
    if (ti >= p.T) return;   // past the last token tile (the host launches full rounds only)
  } else {
    grid_tile(xcd_remap(blockIdx.x, gridDim.x), p.T, p.tt, p.ss, ti, split);
  }
  ti += p.t0;
  const int j0 = (int)((int64_t)split * p.n_vtiles / p.S);
  const int j1 = (int)((int64_t)(split + 1) * p.n_vtiles / p.S);
  const int64_t tok0 = (int64_t)ti * kTile;
  const float k2 = kCapped ? 2.0f * kLog2e * p.logit_scale / p.softcap : 0.0f;
  const float c2 = kCapped ? p.softcap * kLog2e : 0.0f;
  const float l2a = kLog2e * p.logit_scale;

  // Per token column: exponent offset (plain form: with the row class folded
  // in), and in the general form the row scale and Z-loss factor.
  float off[kNI], gsc[kNI], c1[kNI];
  uint32_t col_base[kNI];   // byte offset of (token column, lane's first row) in the G rows
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int col = acc_col(wn, ni, lane);
    const int64_t tok = tok0 + col;
    const bool ok = tok < p.N;
    const int st = ok ? p.row_state[tok] : (int)kRowIgnored;
    const float lse2 = ok ? p.lse[tok] * kLog2e : 0.0f;
    // Capped: + 2 (a factor 4 folded into the exponent; see grad_store_tile).
    const float o = kCapped ? c2 - lse2 + 2.0f : -lse2;
    if (kGen) {
      off[ni] = o;
      gsc[ni] = ok ? p.gs[tok] : 0.0f;
      c1[ni] = ok ? p.c1[tok] : 1.0f;
    } else {
      off[ni] = st == kRowValid ? o : (st == kRowBad ? __builtin_nanf("") : -__builtin_inff());
      gsc[ni] = 1.0f;
      c1[ni] = 1.0f;
    }
    // Blocked G (see DtlKMajorBlockedG): after the lane-half swap of
    // grad_store_tile this lane stores 8 consecutive vocabulary rows of
    // sub-block 2wm + mi/2 at column (mi%2)·32 + 16gp + 8(lane/32) of token
    // row col.
    col_base[ni] = (uint32_t)((2 * wm * kGSubElems + col * kBK + 8 * (lane >> 5)) * 2);
  }
  // The whole token tile, padding rows past N included (they get zeros, which
  // the dW contraction reads).
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.G + (int64_t)ti * p.n_vtiles * kGBlockElems,
                                              p.n_vtiles * kGBlockElems * 2);
  const __amdgpu_buffer_rsrc_t rs_lo =
      kSplit ? make_rsrc(p.G_lo + (int64_t)ti * p.n_vtiles * kGBlockElems, p.n_vtiles * kGBlockElems * 2)
             : rs;

  // Chunk-local tiles j < j_mid lie below V; the tile that reaches past V (at
  // most one) runs in a loop of its own with the masked store.
  const int64_t full_local = (p.V - p.v_begin) / kTile;
  const int j_mid = (int)(j1 < full_local ? j1 : (j0 > full_local ? j0 : full_local));
  const int lrow = acc_row_lane(wm, lane);
  // (The first tile's prologue barrier orders these LDS writes before any read.)
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) s_cand[ni][tid] = 0u;
  if (tid == 0) {
    s_dom[0] = reinterpret_cast<int64_t>(p.dom_base);
    s_dom[1] = p.v_begin + p.key_offset;
  }
  // Cross-tile prefetch as in the forward; the G stores between two tiles
  // make a preloaded tile wait for all outstanding memory operations.
  Sweep sw;
  f32x16 acc[kMI][kNI];
  for (int j = j0; j < j_mid; ++j) {
    const int64_t vloc0 = (int64_t)j * kTile;      // chunk-local vocabulary row
    gemm_tile<false, false, kTail, true, true>(p.W, p.H, p.v_begin + vloc0, p.V, p.X, p.H, tok0, p.N,
                                               0, p.H, p.H, smem, acc, &sw,
                                               j + 1 < j1 ? p.v_begin + vloc0 + kTile : -1);
    uint32_t cb[kNI];
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) cb[ni] = col_base[ni] + (uint32_t)(j * kGBlockElems * 2);
    float pmax[kNI] = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool act = grad_store_tile<kCapped, false, kGen, kFilter, kSplit>(
        acc, off, gsc, c1, p.eps_over_v, rs, rs_lo, cb, 0, k2, c2, l2a, p.filter_eps, pmax);
    grad_mark_candidates<kCapped>(pmax, s_cand, tid, j);
    if (kFilter) store_filter_flag(p.flags, act, ti, j, p.n_vtiles, wave, lane);
  }
  for (int j = j_mid; j < j1; ++j) {
    const int64_t vloc0 = (int64_t)j * kTile;
    const int64_t v0 = p.v_begin + vloc0;
    gemm_tile<false, false, kTail, true, true>(p.W, p.H, v0, p.V, p.X, p.H, tok0, p.N, 0, p.H, p.H,
                                               smem, acc, &sw, j + 1 < j1 ? v0 + kTile : -1);
    uint32_t cb[kNI];
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) cb[ni] = col_base[ni] + (uint32_t)(j * kGBlockElems * 2);
    const int lim = (int)(p.V - v0) - lrow;
    float pmax[kNI] = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool act = grad_store_tile<kCapped, true, kGen, kFilter, kSplit>(
        acc, off, gsc, c1, p.eps_over_v, rs, rs_lo, cb, lim, k2, c2, l2a, p.filter_eps, pmax);
    grad_mark_candidates<kCapped>(pmax, s_cand, tid, j);
    if (kFilter) store_filter_flag(p.flags, act, ti, j, p.n_vtiles, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();   // s_dom, written by thread 0, is read by every thread
  grad_store_candidates(s_cand, s_dom, tid, ti, wn, lane, lrow);
}

// ---------------------------------------------------------------------------
// Row-chunked forward that also keeps every logit of the chunk (the FLCE
// pipeline of Liger as the blog "最贵的一层：深入浅出 Liger Kernel 与 Cut
// Cross-Entropy" describes it in §二: the chunk's logits are formed, the loss
// comes from an online softmax over them, and the gradient is written in
// their place).  The sweep is the forward's: per (token tile, split) a
// running (m, s) over the split's vocabulary tiles, written as one partial
// per token and split.  In the same epilogue each logit is stored as
// U = 2^(u − ref)·d in bf16 (u the base-2 logit, d the softcap derivative),
// the exponential shared with the running sum.  The reference is the running
// max of the lane pair after the tile (kPlain, kCapGeneral; stored per
// 128-column block for the later rescale) or the fixed c2 (kCapFixed).
// U lies in [0, 1]; U·2^(ref − lse) is the softmax times d.
// ---------------------------------------------------------------------------
// Also the candidate of a dominant entry: the lane's largest logit of each
// token column so far in the split and the W row of the lane's first row of
// the tile that held it (cz, cbase in LDS, [ni][thread]; row0 is that row for
// this tile).  A later pass keeps the split's best, and once the LSE is known
// the exact-entry kernel decides whether it is dominant.
template <int kMode, bool kMasked, bool kZSum>
__device__ __forceinline__ void flce_fold_store_tile(const f32x16 (&acc)[kMI][kNI], float (&m)[kNI],
                                                     float (&s)[kNI], float (&zs)[kNI], int lim,
                                                     float k2, float c2, float l2a,
                                                     __amdgpu_buffer_rsrc_t rs,
                                                     const uint32_t (&cb)[kNI],
                                                     float (*cz)[kThreads], int32_t (*cbase)[kThreads],
                                                     int tid, int32_t row0) {
  const float NEG_INF = -__builtin_inff();
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    float mref = c2;
    float zown = NEG_INF;   // the lane's largest logit of the column in this tile
    if (kMode != kCapFixed) {
      float zmax = NEG_INF;
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float z = acc[mi][ni][r];
          zmax = fmaxf(zmax, (!kMasked || acc_row_const(mi, r) < lim) ? z : NEG_INF);
        }
      zown = zmax;
      // One reference for both lanes of the token column, so that a 128-row
      // block of U has a single scale.
      zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
      const float umax = kMode == kPlain ? zmax * l2a
                                         : (zmax == NEG_INF ? NEG_INF : c2 * tanh_of_scaled(zmax, k2));
      const float mn = fmaxf(m[ni], umax);
      mref = mn == NEG_INF ? 0.0f : mn;
      s[ni] *= exp2_fast(m[ni] - mref);
      m[ni] = mn;
    }
    float sum = 0.0f, zsum = 0.0f;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        u32x2 pk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int gq = 2 * gp + h;
          float uv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = gq * 4 + q;
            const float z = acc[mi][ni][r];
            const bool ok = !kMasked || acc_row_const(mi, r) < lim;
            if (kMode == kCapFixed) zown = fmaxf(zown, ok ? z : NEG_INF);
            float e, u, zt;
            if (kMode == kPlain) {
              e = exp2_fast(fmaf(z, l2a, -mref));
              u = e;
              zt = z;
            } else {
              const float rr = rcp_fast(exp2_fast(z * k2) + 1.0f);
              const float d4 = 4.0f * rr;
              const float d = fmaf(-d4, rr, d4);                  // 1 − tanh² = 4r(1 − r)
              e = kMode == kCapFixed ? exp2_fast(-2.0f * c2 * rr)  // 2^(c2·tanh − c2)
                                     : exp2_fast(fmaf(-2.0f * c2, rr, c2 - mref));
              u = e * d;
              zt = fmaf(-2.0f, rr, 1.0f);                         // tanh = 1 − 2r
            }
            sum += ok ? e : 0.0f;
            if (kZSum) zsum += ok ? zt : 0.0f;
            uv[q] = ok ? u : 0.0f;
          }
          pk[h][0] = pack_bf16x2(uv[0], uv[1]);
          pk[h][1] = pack_bf16x2(uv[2], uv[3]);
        }
        // Blocked layout, 8 rows per lane after the lane-half swap (as the
        // recompute path's gradient chunk, grad_store_tile).
        const auto s0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
        const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
        const uint32_t eo = (uint32_t)((mi >> 1) * kGSubElems + (mi & 1) * 32 + 16 * gp);
        __builtin_amdgcn_raw_buffer_store_b128(out, rs, (int)(cb[ni] + 2u * eo), 0, 0);
      }
    s[ni] += sum;
    if (kZSum) zs[ni] += zsum;
    if (zown > cz[ni][tid]) {
      cz[ni][tid] = zown;
      cbase[ni][tid] = row0;
    }
  }
}

// End of a fused sweep: the split's dominant-entry candidate of each token,
// the best of the four lanes that hold its column (lanes l and l^32 of the
// two waves with the same wn), the larger logit first, then the smaller row.
__device__ __forceinline__ void flce_store_candidates(const float (*cz)[kThreads],
                                                      const int32_t (*cbase)[kThreads], int wm,
                                                      int wn, int lane, int64_t tok0, int split,
                                                      int64_t N, float* part_cz, int32_t* part_cb) {
  __syncthreads();
  if (wm != 0 || lane >= 32) return;
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t tok = tok0 + acc_col(wn, ni, lane);
    if (tok >= N) continue;
    const int t0 = wn * 64 + lane, t1 = (2 + wn) * 64 + lane;
    const int holders[4] = {t0, t0 + 32, t1, t1 + 32};
    float bz = cz[ni][holders[0]];
    int32_t bb = cbase[ni][holders[0]];
#pragma unroll
    for (int h = 1; h < 4; ++h) {
      const float z = cz[ni][holders[h]];
      const int32_t b = cbase[ni][holders[h]];
      if (z > bz || (z == bz && b >= 0 && (bb < 0 || b < bb))) {
        bz = z;
        bb = b;
      }
    }
    part_cz[(int64_t)split * N + tok] = bz;
    part_cb[(int64_t)split * N + tok] = bb;
  }
}

// Reference of tile j for the wave's 128-row half, through the descriptor
// `rr` of the ref rows tok0.. (rows past N are out of range).  Lanes l and
// l^32 hold the same value after the fold's pair max and store it to the
// same address.
__device__ __forceinline__ void flce_store_ref(__amdgpu_buffer_rsrc_t rr, uint32_t ref_base,
                                               const float (&m)[kNI], int j, int wm,
                                               uint32_t ni_stride) {
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni)
    buffer_store_f32(m[ni], rr, ref_base + ni * ni_stride + (uint32_t)(2 * j + wm) * 4u);
}

template <bool kTail, int kMode, bool kZSum>
__global__ void __launch_bounds__(kThreads, 1)
flce_logits_kernel(FlceParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[4 * kStageElems];
  __shared__ float s_cz[kNI][kThreads];      // dominant-entry candidates (see
  __shared__ int32_t s_cb[kNI][kThreads];    // flce_fold_store_tile)
  LCE_LDS uint16_t* smem = (LCE_LDS uint16_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  int ti, split;
  grid_tile(g, p.T, p.tt, p.ss, ti, split);
  const int j0 = (int)((int64_t)split * p.n_vtiles / p.S);
  const int j1 = (int)((int64_t)(split + 1) * p.n_vtiles / p.S);
  const int64_t tok0 = (int64_t)ti * kTile;
  const float k2 = kMode != kPlain ? 2.0f * kLog2e * p.logit_scale / p.softcap : 0.0f;
  const float c2 = kMode != kPlain ? p.softcap * kLog2e : 0.0f;
  const float l2a = kLog2e * p.logit_scale;
  const int nref = 2 * p.n_vtiles;

  float m[kNI], s[kNI], zs[kNI];
  uint32_t col_base[kNI];   // byte offset of (token column, lane's first row) in the U rows
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    m[ni] = kMode == kCapFixed ? c2 : -__builtin_inff();
    s[ni] = 0.0f;
    zs[ni] = 0.0f;
    col_base[ni] = (uint32_t)((2 * wm * kGSubElems + acc_col(wn, ni, lane) * kBK + 8 * (lane >> 5)) * 2);
    s_cz[ni][tid] = -__builtin_inff();
    s_cb[ni][tid] = -1;
  }
  const int lrow = acc_row_lane(wm, lane);
  // U is blocked like the recompute path's gradient chunk: the token tile's
  // n_vtiles blocks, rows past N included (their values are finite and meet
  // only zero rows of X in the dW contraction).
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.U + (int64_t)ti * p.n_vtiles * kGBlockElems,
                                              p.n_vtiles * kGBlockElems * 2);
  // ref rows tok0 .. N − 1 (unused with the fixed reference).
  const __amdgpu_buffer_rsrc_t rr =
      make_rsrc(kMode != kCapFixed ? p.ref + tok0 * nref : p.part_m, kMode != kCapFixed ? (p.N - tok0) * nref * 4 : 0);
  const uint32_t ref_base = (uint32_t)(acc_col(wn, 0, lane) * nref * 4);
  const uint32_t ref_ni_stride = (uint32_t)(32 * nref * 4);   // 32 token columns per ni

  const int j_mid = (int)(j1 < p.V / kTile ? j1 : (j0 > p.V / kTile ? j0 : p.V / kTile));
  Sweep sw;
  f32x16 acc[kMI][kNI];
  // Tiles below V, then (in a loop of its own, as in the forward) the one
  // tile that reaches past V.
  for (int j = j0; j < j_mid; ++j) {
    const int64_t v0 = (int64_t)j * kTile;
    gemm_tile<false, false, kTail, true, true>(p.W, p.H, v0, p.V, p.X, p.H, tok0, p.N, 0, p.H,
                                               p.H, smem, acc, &sw, j + 1 < j1 ? v0 + kTile : -1);
    uint32_t cb[kNI];
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) cb[ni] = col_base[ni] + (uint32_t)(j * kGBlockElems * 2);
    flce_fold_store_tile<kMode, false, kZSum>(acc, m, s, zs, 0, k2, c2, l2a, rs, cb, s_cz, s_cb, tid,
                                              (int32_t)(v0 + lrow));
    if (kMode != kCapFixed) flce_store_ref(rr, ref_base, m, j, wm, ref_ni_stride);
  }
  for (int j = j_mid; j < j1; ++j) {
    const int64_t v0 = (int64_t)j * kTile;
    gemm_tile<false, false, kTail, true, true>(p.W, p.H, v0, p.V, p.X, p.H, tok0, p.N, 0, p.H,
                                               p.H, smem, acc, &sw, j + 1 < j1 ? v0 + kTile : -1);
    uint32_t cb[kNI];
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) cb[ni] = col_base[ni] + (uint32_t)(j * kGBlockElems * 2);
    const int lim = (int)(p.V - v0) - lrow;
    flce_fold_store_tile<kMode, true, kZSum>(acc, m, s, zs, lim, k2, c2, l2a, rs, cb, s_cz, s_cb, tid,
                                             (int32_t)(v0 + lrow));
    if (kMode != kCapFixed) flce_store_ref(rr, ref_base, m, j, wm, ref_ni_stride);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  store_split_partials<kMode, kZSum>(m, s, zs, reinterpret_cast<float*>(smem_raw), wm, wn, lane,
                                     tok0, split, p.N, p.N,
                                     kMode == kPlain ? p.logit_scale : p.softcap, p.part_m,
                                     p.part_s, p.part_z);
  flce_store_candidates(s_cz, s_cb, wm, wn, lane, tok0, split, p.N, p.part_cz, p.part_cb);
}

// ---------------------------------------------------------------------------
// Backward, steps 2 and 3 for one vocabulary chunk, in one persistent launch.
//
//   dX tile (256 tokens x 256 hidden): dX_acc (+)= G[:, chunk] · W[chunk, :]
//     M = tokens (A = G, K-major), N = hidden (B = W chunk, MN-major: its rows
//     are vocabulary entries, i.e. K); G is zero past V and W reads past V
//     return 0.  (AI-infra KB M011 §06: dH accumulates dZ · W over the
//     vocabulary tiles.)
//   dW tile (256 vocabulary x 256 hidden): dW[v] = s · Σ_tok G[tok][v]·x_tok
//     M = chunk vocabulary (A = G, MN-major), N = hidden (B = X, MN-major),
//     K = tokens, rows past N read as zero.  (M011 §06: dW += dZᵀ · H.)
//
// Schedule: kXcds x kCusPerXcd workgroups, one per compute unit; workgroup b
// runs on XCD b % kXcds.  Each XCD owns a contiguous range of dX tile ids and
// of dW tile ids (neighbouring ids share G, W and X slices in its L2).  Inside
// an XCD the kind of tile with more K steps (dX: the chunk's vocabulary; dW:
// the tokens) is dealt round-robin, so the first rl workgroups hold one more
// of it; the other kind is dealt round-robin as well, the rl heavier
// workgroups taking only what balances the cost (K steps) of the two groups.
// Concurrent workgroups therefore work on consecutive tile ids, and every
// tile has exactly one owner, so the read-modify-writes need no
// synchronisation.
// ---------------------------------------------------------------------------
// dX tile id g = part · (nt_tok · nt_h) + tile: K steps [part·D, (part+1)·D)
// of the chunk, D = ceil(steps / ksplit), into partial buffer `part`.  The
// host picks ksplit so that every part holds at least one step.
template <bool kFilter>
__device__ __forceinline__ void chunk_dx_tile(const ChunkGemmParams& p, int g, int64_t D,
                                              LCE_LDS uint16_t* smem, int wm, int wn, int lane) {
  const int64_t lda = p.nt_v;   // blocked G: its reader takes the count of vocabulary tiles
  f32x16 acc[kMI][kNI];
  zero_acc(acc);
  const int n_tiles = p.nt_tok * p.nt_h;
  const int part = g / n_tiles;
  const int t = g - part * n_tiles;
  const int64_t tok0 = (int64_t)(t / p.nt_h) * kTile;
  const int64_t h0 = (int64_t)(t % p.nt_h) * kTile;
  const int64_t steps = (p.chunk_len + kBK - 1) / kBK;
  const int64_t k0 = (int64_t)part * D * kBK;
  const int64_t k_end = (part + 1) * D < steps ? (part + 1) * D * kBK : steps * kBK;
  if (kFilter) {
    // Gradient filter (one K part): only the runs of vocabulary tiles with a
    // value above the threshold for this token tile.
    // Every value here is wave-uniform (kept in scalar registers).
    const uint32_t* fr = p.flags + (int64_t)(t / p.nt_h) * p.nt_v;
    const int nv = p.nt_v;
    int j = 0;
    while (true) {
      while (j < nv && __builtin_amdgcn_readfirstlane(fr[j]) == 0u) ++j;
      if (j >= nv) break;
      const int ja = j;
      while (j < nv && __builtin_amdgcn_readfirstlane(fr[j]) != 0u) ++j;
      const int64_t kb = (int64_t)j * kTile < k_end ? (int64_t)j * kTile : k_end;
      gemm_tile<false, true, false, false, false, true>(p.G, lda, tok0, p.N, p.Wc, p.H, h0, p.H,
                                                         (int64_t)ja * kTile, kb, p.wc_rows, smem,
                                                         acc);
    }
  } else {
    gemm_tile<false, true, false, false, false, true>(p.G, lda, tok0, p.N, p.Wc, p.H, h0, p.H, k0,
                                                       k_end, p.wc_rows, smem, acc);
  }
  // dX_acc rows tok0.. through a descriptor that ends at row N; columns at or
  // past H are pushed out of range.  The 64 previous values of one mi row
  // block are loaded together, so a tile costs 4 round trips, not 256.
  float* dst = p.dX_acc + (int64_t)part * p.dx_part_stride;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(dst + tok0 * p.H, (p.N - tok0) * p.H * 4);
  const uint32_t rowb = (uint32_t)(p.H * 4);
  uint32_t cbase[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t h = h0 + acc_col(wn, ni, lane);
    cbase[ni] = h < p.H ? (uint32_t)acc_row_lane(wm, lane) * rowb + (uint32_t)h * 4u : kOutOfRange;
  }
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) {
    float prev[kNI][16];
    if (p.accumulate) {
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          prev[ni][r] = buffer_load_f32(rs, cbase[ni] + (uint32_t)acc_row_const(mi, r) * rowb);
    } else {
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) prev[ni][r] = 0.0f;
    }
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        buffer_store_f32(prev[ni][r] + acc[mi][ni][r], rs,
                         cbase[ni] + (uint32_t)acc_row_const(mi, r) * rowb);
  }
}

template <bool kDwAcc, bool kFilter>
__device__ __forceinline__ void chunk_dw_tile(const ChunkGemmParams& p, int g, float sc,
                                              LCE_LDS uint16_t* smem, int wm, int wn, int lane) {
  const int64_t lda = p.nt_v;   // blocked G: its reader takes the count of vocabulary tiles
  f32x16 acc[kMI][kNI];
  zero_acc(acc);
  const int64_t vt0 = (int64_t)(g / p.nt_h) * kTile;
  const int64_t h0 = (int64_t)(g % p.nt_h) * kTile;
  if (kFilter) {
    // Gradient filter: only the runs of token tiles with a value above the
    // threshold in this vocabulary tile.
    const uint32_t* fc = p.flags + g / p.nt_h;
    const int nt = p.nt_tok, nv = p.nt_v;
    int t = 0;
    while (true) {
      while (t < nt && __builtin_amdgcn_readfirstlane(fc[(int64_t)t * nv]) == 0u) ++t;
      if (t >= nt) break;
      const int ta = t;
      while (t < nt && __builtin_amdgcn_readfirstlane(fc[(int64_t)t * nv]) != 0u) ++t;
      const int64_t kb = (int64_t)t * kTile < p.N ? (int64_t)t * kTile : p.N;
      gemm_tile<true, true, false, false, false, true>(p.G, lda, vt0, p.ldg, p.X, p.H, h0, p.H,
                                                        (int64_t)ta * kTile, kb, p.N, smem, acc);
    }
  } else {
    gemm_tile<true, true, false, false, false, true>(p.G, lda, vt0, p.ldg, p.X, p.H, h0, p.H, 0,
                                                      p.N, p.N, smem, acc);
  }
  // dW rows vt0.. of the chunk through a descriptor that ends at chunk_len;
  // columns at or past H are pushed out of range.
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.dW_dst + vt0 * p.H, (p.chunk_len - vt0) * p.H * 4);
  const uint32_t rowb = (uint32_t)(p.H * 4);
  uint32_t cbase[kNI];
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) {
    const int64_t h = h0 + acc_col(wn, ni, lane);
    cbase[ni] = h < p.H ? (uint32_t)acc_row_lane(wm, lane) * rowb + (uint32_t)h * 4u : kOutOfRange;
  }
  if (kDwAcc) {
    // Read-modify-write, the 64 previous values of one mi row block together.
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
      float prev[kNI][16];
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          prev[ni][r] = buffer_load_f32(rs, cbase[ni] + (uint32_t)acc_row_const(mi, r) * rowb);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          buffer_store_f32(fmaf(sc, acc[mi][ni][r], prev[ni][r]), rs,
                           cbase[ni] + (uint32_t)acc_row_const(mi, r) * rowb);
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          buffer_store_f32(sc * acc[mi][ni][r], rs, cbase[ni] + (uint32_t)acc_row_const(mi, r) * rowb);
  }
}

template <bool kDwAcc, bool kFilter>
__global__ void __launch_bounds__(kThreads, 1)
chunk_gemm_kernel(ChunkGemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[4 * kStageElems];
  LCE_LDS uint16_t* smem = (LCE_LDS uint16_t*)smem_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int xcd = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
  const int n_dx = p.nt_tok * p.nt_h * p.ksplit, n_dw = p.nt_v * p.nt_h;
  const int dx_lo = (int)((int64_t)xcd * n_dx / kXcds);
  const int nx = (int)((int64_t)(xcd + 1) * n_dx / kXcds) - dx_lo;
  const int dw_lo = (int)((int64_t)xcd * n_dw / kXcds);
  const int nw = (int)((int64_t)(xcd + 1) * n_dw / kXcds) - dw_lo;
  // Cost of a tile in K steps: D for dX tiles (one K part), E for dW tiles.
  const int64_t D = ((p.chunk_len + kBK - 1) / kBK + p.ksplit - 1) / p.ksplit;
  const int64_t E = (p.N + kBK - 1) / kBK;
  // The longer kind of tile is dealt first, round-robin; the workgroups that
  // hold one more of it (the first rl, "heavy") take h of the shorter kind
  // each and the others share the rest, with h chosen so that the larger of
  // the two groups' K steps per workgroup is least.  (Values are uniform over
  // the workgroup: a scalar loop of at most ns_t / rl + 1 steps.)
  const bool dw_long = E > D;
  const int nl_t = dw_long ? nw : nx, ns_t = dw_long ? nx : nw;
  const int64_t cl = dw_long ? E : D, cs = dw_long ? D : E;
  const int rl = nl_t % kCusPerXcd;
  int ns_heavy = 0;
  if (rl > 0) {
    const int64_t load_h = (int64_t)(nl_t / kCusPerXcd + 1) * cl, load_l = load_h - cl;
    const int n_light = kCusPerXcd - rl;
    int64_t best = -1;
    for (int h = 0;; ++h) {
      const int c = rl * h < ns_t ? rl * h : ns_t;
      const int64_t heavy = load_h + (int64_t)h * cs;
      const int64_t light = load_l + (int64_t)((ns_t - c + n_light - 1) / n_light) * cs;
      const int64_t load = heavy > light ? heavy : light;
      if (best < 0 || load < best) {
        best = load;
        ns_heavy = c;
      }
      if (c >= ns_t) break;
    }
  }
  const int ns_light = ns_t - ns_heavy;
  const float sc = *p.scale;

  // This workgroup's share of each kind: ids start, start + stride, ... below
  // limit, after `offset` (long kind: round-robin; short kind: the light
  // workgroups share the first ns_light ids, the heavy ones the rest).
  int l_start = li, l_stride = kCusPerXcd, l_limit = nl_t;
  int s_start, s_stride, s_limit, s_offset = 0;
  if (li >= rl) {
    s_start = li - rl; s_stride = kCusPerXcd - rl; s_limit = ns_light;
  } else {
    s_start = li; s_stride = rl; s_limit = ns_heavy; s_offset = ns_light;
  }
  const int x_start = dw_long ? s_start : l_start, x_stride = dw_long ? s_stride : l_stride;
  const int x_limit = dw_long ? s_limit : l_limit, x_offset = dw_long ? s_offset : 0;
  const int w_start = dw_long ? l_start : s_start, w_stride = dw_long ? l_stride : s_stride;
  const int w_limit = dw_long ? l_limit : s_limit, w_offset = dw_long ? 0 : s_offset;
  for (int t = x_start; t < x_limit; t += x_stride)
    chunk_dx_tile<kFilter>(p, dx_lo + x_offset + t, D, smem, wm, wn, lane);
  for (int t = w_start; t < w_limit; t += w_stride)
    chunk_dw_tile<kDwAcc, kFilter>(p, dw_lo + w_offset + t, sc, smem, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_lse_partials(const LseParams& p, hipStream_t stream) {
  const int grid = p.T * p.S;
  const bool tail = p.H % kBK != 0, zsum = p.part_z != nullptr;
  // Fixed reference 2^(u - c2) >= 2^(-2·c2) stays a normal float for c2 < 60.
  const int mode = p.softcap <= 0.0f ? kPlain
                   : (p.softcap * kLog2e < 60.0f ? kCapFixed : kCapGeneral);
#define LCE_LSE_LAUNCH(T_, M_, Z_) \
  hipLaunchKernelGGL((lse_partials_kernel<T_, M_, Z_>), dim3(grid), dim3(kThreads), 0, stream, p)
#define LCE_LSE_MODES(T_, Z_)                          \
  do {                                                 \
    if (mode == kPlain) LCE_LSE_LAUNCH(T_, kPlain, Z_);     \
    else if (mode == kCapFixed) LCE_LSE_LAUNCH(T_, kCapFixed, Z_); \
    else LCE_LSE_LAUNCH(T_, kCapGeneral, Z_);          \
  } while (0)
  if (tail) {
    if (zsum) LCE_LSE_MODES(true, true);
    else LCE_LSE_MODES(true, false);
  } else {
    if (zsum) LCE_LSE_MODES(false, true);
    else LCE_LSE_MODES(false, false);
  }
#undef LCE_LSE_MODES
#undef LCE_LSE_LAUNCH
  return hipGetLastError();
}

bool flce_fixed_reference(float softcap) { return softcap > 0.0f && softcap * kLog2e < 60.0f; }

hipError_t launch_flce_logits(const FlceParams& p, hipStream_t stream) {
  const int grid = p.T * p.S;
  const bool tail = p.H % kBK != 0, zsum = p.part_z != nullptr;
  const int mode = p.softcap <= 0.0f ? kPlain
                   : (flce_fixed_reference(p.softcap) ? kCapFixed : kCapGeneral);
#define LCE_FLCE_LAUNCH(T_, M_, Z_) \
  hipLaunchKernelGGL((flce_logits_kernel<T_, M_, Z_>), dim3(grid), dim3(kThreads), 0, stream, p)
#define LCE_FLCE_MODES(T_, Z_)                               \
  do {                                                       \
    if (mode == kPlain) LCE_FLCE_LAUNCH(T_, kPlain, Z_);       \
    else if (mode == kCapFixed) LCE_FLCE_LAUNCH(T_, kCapFixed, Z_); \
    else LCE_FLCE_LAUNCH(T_, kCapGeneral, Z_);               \
  } while (0)
  // Σ z only serves label smoothing, which the fused call takes without a
  // softcap only.
  if (zsum && mode != kPlain) return hipErrorInvalidValue;
  if (tail) {
    if (zsum) LCE_FLCE_LAUNCH(true, kPlain, true);
    else LCE_FLCE_MODES(true, false);
  } else {
    if (zsum) LCE_FLCE_LAUNCH(false, kPlain, true);
    else LCE_FLCE_MODES(false, false);
  }
#undef LCE_FLCE_MODES
#undef LCE_FLCE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_grad_logits(const GradParams& p, hipStream_t stream) {
  const int per_round = kXcds * kCusPerXcd;
  if (p.round_tiles > 0 && (p.round_tiles % kXcds != 0 || p.round_tiles * p.S != per_round))
    return hipErrorInvalidValue;
  const int grid = p.round_tiles > 0 ? (p.T + p.round_tiles - 1) / p.round_tiles * per_round
                                     : p.T * p.S;
  const bool tail = p.H % kBK != 0, capped = p.softcap > 0.0f, gen = p.gs != nullptr;
  const bool filt = p.flags != nullptr, split = p.G_lo != nullptr;
  if (!p.dom_base || (filt && split)) return hipErrorInvalidValue;
#define LCE_GRAD_LAUNCH(T_, C_, G_, F_, S_) \
  hipLaunchKernelGGL((grad_logits_kernel<T_, C_, G_, F_, S_>), dim3(grid), dim3(kThreads), 0, stream, p)
#define LCE_GRAD_TC(G_, F_, S_)                                   \
  do {                                                            \
    if (tail && capped) LCE_GRAD_LAUNCH(true, true, G_, F_, S_);  \
    else if (tail) LCE_GRAD_LAUNCH(true, false, G_, F_, S_);      \
    else if (capped) LCE_GRAD_LAUNCH(false, true, G_, F_, S_);    \
    else LCE_GRAD_LAUNCH(false, false, G_, F_, S_);               \
  } while (0)
  if (filt) {
    if (gen) LCE_GRAD_TC(true, true, false);
    else LCE_GRAD_TC(false, true, false);
  } else if (split) {
    if (gen) LCE_GRAD_TC(true, false, true);
    else LCE_GRAD_TC(false, false, true);
  } else {
    if (gen) LCE_GRAD_TC(true, false, false);
    else LCE_GRAD_TC(false, false, false);
  }
#undef LCE_GRAD_TC
#undef LCE_GRAD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_chunk_gemm(const ChunkGemmParams& p, hipStream_t stream) {
  const int grid = kXcds * kCusPerXcd;
  // The filtered form reads one flag word per tile and K part; it serves the
  // recompute path only (one K part, dW written once).
  if (p.flags && (p.ksplit != 1 || p.dw_accumulate)) return hipErrorInvalidValue;
  if (p.flags)
    hipLaunchKernelGGL((chunk_gemm_kernel<false, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if (p.dw_accumulate)
    hipLaunchKernelGGL((chunk_gemm_kernel<true, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((chunk_gemm_kernel<false, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lce
