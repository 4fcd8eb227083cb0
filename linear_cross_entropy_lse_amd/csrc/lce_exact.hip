// Exact entries of the backward's logit gradient (see launch_exact_entries in
// lce_internal.h).
//
// The gradient of a row is softmax − onehot (blog "最贵的一层：深入浅出 Liger
// Kernel 与 Cut Cross-Entropy", §二; AI-infra KB M011 §06), times the softcap
// derivative (Unsloth fused cross-entropy chapter, §4).  The backward carries
// its softmax part through a bf16 chunk.  Two entries per row are taken out of
// that chunk and applied in fp32 instead:
//   * the label's entry: when a row predicts its label confidently, p·d there
//     nearly cancels the one-hot term d, so the true entry d·(p − 1) is far
//     below the bf16 rounding of p·d;
//   * an entry with softmax above 1/2 + 2^-10 (at most one per row): it alone
//     carries a large share of the row's gradient, which bf16 would round at
//     2^-9 of that share.
// The value of an entry is formed from its logit exactly as the tile kernels
// form it (grad_value); the logit is recomputed here with the same sequence of
// v_mfma_f32_32x32x16_bf16 over K as the tile kernels use, so it is the value
// the forward's LSE and the logit-gradient tile saw, bit for bit.  That keeps
// p − 1 of a confident row at the size the LSE itself implies.
// The backward computes the label entries' values once, over the whole
// vocabulary; after each chunk's logit-gradient pass it only writes their
// slots in G (the labels of a chunk are one run of the label-sorted keys) and
// takes the dominant entries the pass marked.
#include "lce_device.h"
#include "lce_internal.h"

namespace lce {
namespace {

constexpr int kExactRows = 32;   // token rows per wave (one MFMA column block)

__device__ __forceinline__ bf16x8 load8(const uint16_t* row, int64_t k, int64_t H) {
  if (k >= H) return bf16x8{};
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + k));
}

// C = A·Bᵀ for one 32 x 32 block over K = H in 16-deep slices: lane l feeds A
// row (l % 32) and B row (l % 32), K values 8·(l / 32) .. +7 of each slice
// (null rows feed zeros).  The same products in the same order as the tile
// kernels' MFMA chains for these (row, column) pairs.  The fragments of
// kBatch slices are loaded before their MFMAs, and the next batch's loads are
// in flight while a batch multiplies, so the chain is not bound by the
// latency of its loads.
constexpr int kBatch = 8;

__device__ __forceinline__ f32x16 block_logits(const uint16_t* arow, const uint16_t* brow,
                                               int64_t H, int lane) {
  f32x16 acc = {};
  const int64_t kh = 8 * (lane >> 5);
  bf16x8 a[2][kBatch], b[2][kBatch];
  auto load = [&](int buf, int64_t k0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t k = k0 + 16 * u + kh;
      a[buf][u] = arow ? load8(arow, k, H) : bf16x8{};
      b[buf][u] = brow ? load8(brow, k, H) : bf16x8{};
    }
  };
  // Slices past H hold zeros only; adding their 0·0 products would leave acc
  // as it is, so they are skipped.
  auto mma = [&](int buf, int64_t k0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (k0 + 16 * u < H)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[buf][u], b[buf][u], acc, 0, 0, 0);
  };
  const int64_t step = 16 * kBatch;
  load(0, 0);
  for (int64_t k0 = 0; k0 < H; k0 += 2 * step) {
    if (k0 + step < H) load(1, k0 + step);
    mma(0, k0);
    if (k0 + step < H) {
      if (k0 + 2 * step < H) load(0, k0 + 2 * step);
      mma(1, k0 + step);
    }
  }
  return acc;
}

// Element r of lane l of a 32 x 32 MFMA block holds C[8(r/4) + 4(l/32) + r%4][l % 32].
__device__ __forceinline__ float pick(const f32x16& c, int r) {
  float v = c[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) v = r == k ? c[k] : v;
  return v;
}

// Byte-free element offset of (token, chunk-local column) in the blocked G.
__device__ __forceinline__ int64_t g_offset(int64_t tok, int64_t col, int n_vtiles) {
  return ((tok / kTile) * n_vtiles + col / kTile) * kGBlockElems + ((col % kTile) / kBK) * kGSubElems +
         (tok % kTile) * kBK + col % kBK;
}

// A token row's terms, as the logit-gradient kernel forms them: exponent
// offset (plain form: with the row class folded in), row scale, Z-loss
// factor, whether the row has a gradient, and the value G holds for a logit
// of −inf there (0, or −gsc·e/V without softcap) with its lo part.
struct RowTerms {
  float o, off, gsc, c1;
  bool live;
  uint16_t vinf_bits, vinf_lo;
  float vinf;
};

template <bool kCapped, bool kGen>
__device__ __forceinline__ RowTerms row_terms(const ExactParams& p, int64_t tok, float c2) {
  RowTerms t;
  const bool in = tok >= 0 && tok < p.N;
  const int st = in ? p.row_state[tok] : (int)kRowIgnored;
  const float lse2 = in ? p.lse[tok] * kLog2e : 0.0f;
  t.o = kCapped ? c2 - lse2 + 2.0f : -lse2;
  if (kGen) {
    t.off = t.o;
    t.gsc = in ? p.gs[tok] : 0.0f;
    t.c1 = in ? p.c1[tok] : 1.0f;
    t.live = t.gsc != 0.0f && t.gsc == t.gsc;
  } else {
    t.off = st == kRowValid ? t.o : (st == kRowBad ? __builtin_nanf("") : -__builtin_inff());
    t.gsc = 1.0f;
    t.c1 = 1.0f;
    t.live = st == kRowValid;
  }
  t.vinf = (!kCapped && kGen) ? -t.gsc * p.eps_over_v : 0.0f;
  t.vinf_bits = (uint16_t)f32_to_bf16_bits(t.vinf);
  t.vinf_lo = (uint16_t)f32_to_bf16_bits(t.vinf - bf16_bits_to_f32(t.vinf_bits));
  // In the fused call's stored logits the slot gets the logit value whose
  // image under the later rescale (G = f·U − gs·e/V) is vinf: 0.
  if (p.g_logits) t.vinf_bits = t.vinf_lo = 0;
  return t;
}

template <bool kCapped, bool kGen>
__global__ void __launch_bounds__(64)
exact_entries_kernel(ExactParams p) {
  const int lane = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kExactRows;
  const float k2 = kCapped ? 2.0f * kLog2e * p.logit_scale / p.softcap : 0.0f;
  const float c2 = kCapped ? p.softcap * kLog2e : 0.0f;
  const float l2a = kLog2e * p.logit_scale;
  const int64_t c_lo = p.v_begin, c_hi = p.v_begin + p.chunk_len;

  // ---- the label's entry: the block's diagonal C[j][j] = x_j · w_{y_j} ----
  const int32_t* row_key = p.row_key;
  if (p.label_pass == kLabelValues) {
    // Tokens t0 .. t0 + 31 in order: their label entries' values, and (with
    // G) the value of a logit at −inf in G there.
    const int64_t ltok = t0 + (lane & 31);
    int64_t lw = -1;
    if (ltok < p.N && p.row_state[ltok] == kRowValid && row_key[ltok] != INT32_MAX)
      lw = (int64_t)row_key[ltok] - p.key_offset;
    const bool lab = lw >= c_lo && lw < c_hi;
    if (__builtin_amdgcn_ballot_w64(lab) != 0) {
      const RowTerms rt = row_terms<kCapped, kGen>(p, lab ? ltok : -1, c2);
      const f32x16 c = block_logits(lab ? p.W + lw * p.H : nullptr,
                                    lab ? p.X + ltok * p.H : nullptr, p.H, lane);
      // Row j = lane % 32 of the diagonal sits in lane half (j / 4) % 2.
      const int j = lane & 31;
      if (lab && ((j >> 2) & 1) == (lane >> 5)) {
        const float z = pick(c, ((j >> 3) & 3) * 4 + (j & 3));
        float pr, d;
        const float val = grad_value<kCapped, kGen>(z, rt.off, rt.gsc, rt.c1, p.eps_over_v, k2,
                                                    c2, l2a, pr, d);
        p.lab_dense[ltok] = val - rt.vinf;
        p.lab_oh[ltok] = (kGen ? rt.gsc : 1.0f) * p.one_minus_eps * d;
        if (p.G) {
          const int64_t g = g_offset(ltok, lw - c_lo, p.n_vtiles);
          p.G[g] = rt.vinf_bits;
          if (p.G_lo) p.G_lo[g] = rt.vinf_lo;
        }
      }
    }
  } else if (p.label_pass == kLabelSlots) {
    // The values are known (an earlier kLabelValues pass over the whole
    // vocabulary); only G's entries at the labels in this chunk are set to
    // the value of a logit at −inf.  Those rows are one run of the
    // label-sorted keys: this wave takes keys t0 .. t0 + 31.
    const int64_t i = t0 + (lane & 31);
    if (i < *p.n_keys) {
      const uint64_t k = p.keys[i];
      const int64_t ltok = (int64_t)(uint32_t)k;
      const int64_t lw = (int64_t)(uint32_t)(k >> 32) - p.key_offset;
      if (lw >= c_lo && lw < c_hi) {
        float vinf = 0.0f;
        if (!kCapped && kGen) vinf = -p.gs[ltok] * p.eps_over_v;
        const uint16_t vb = (uint16_t)f32_to_bf16_bits(vinf);
        const int64_t g = g_offset(ltok, lw - c_lo, p.n_vtiles);
        p.G[g] = vb;
        if (p.G_lo) p.G_lo[g] = (uint16_t)f32_to_bf16_bits(vinf - bf16_bits_to_f32(vb));
      }
    }
  }
  if (!p.dom_base && !p.cand_z) return;   // no dominant entries in this pass

  // This lane's token in token order (column lane % 32 of the block) and its
  // row terms, for the dominant entry.  A wave without a candidate in this
  // chunk stops after reading them.
  const int64_t tok = t0 + (lane & 31);
  const bool in = tok < p.N;
  if (p.dom_base) {
    const int32_t d0 = in ? p.dom_base[tok] : -1;
    const int64_t b0 = d0 < 0 ? -1 : (int64_t)d0 - p.key_offset;
    if (__builtin_amdgcn_ballot_w64(b0 >= c_lo && b0 < c_hi) == 0) return;
  }
  const RowTerms tr = row_terms<kCapped, kGen>(p, tok, c2);
  const float o = tr.o, off = tr.off, gsc = tr.gsc, c1 = tr.c1, vinf = tr.vinf;
  const bool live = tr.live;
  const uint16_t vinf_bits = tr.vinf_bits, vinf_lo = tr.vinf_lo;
  const int32_t key = (in && p.row_state[tok] == kRowValid) ? row_key[tok] : INT32_MAX;
  const int64_t wrow = key == INT32_MAX ? -1 : (int64_t)key - p.key_offset;   // the label's W row

  // ---- a dominant entry: among the 64 rows the finding lane held ----
  const float zthr = dominance_threshold<kCapped>(live, o, k2, c2, l2a);
  int32_t db = -1;
  if (in && live) {
    if (p.dom_base) {
      db = p.dom_base[tok];
    } else {
      // The fused forward's per-split candidates: the largest logit (the
      // smaller row on ties) is dominant if it lies above the threshold.
      float bz = -__builtin_inff();
      int32_t bb = -1;
      for (int sp = 0; sp < p.cand_splits; ++sp) {
        const float z = p.cand_z[(int64_t)sp * p.N + tok];
        const int32_t b = p.cand_b[(int64_t)sp * p.N + tok];
        if (z > bz || (z == bz && b >= 0 && (bb < 0 || b < bb))) {
          bz = z;
          bb = b;
        }
      }
      db = bz > zthr ? bb : -1;
    }
  }
  const int64_t base = db < 0 ? -1 : (int64_t)db - p.key_offset;
  const bool dom = base >= c_lo && base < c_hi;
  uint64_t todo = __builtin_amdgcn_ballot_w64(dom && lane < kExactRows);
  while (todo) {
    const int jt = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int64_t tj = t0 + jt;
    const int64_t bj = (int64_t)__shfl(db, jt) - p.key_offset;
    // Candidate q (0..63) is row bj + x(q), x = 32·(q/16) + 8·((q%16)/4) + q%4
    // (the lane's rows of a 256-row tile); two blocks of 32, all columns the
    // token's x.
    float best = -__builtin_inff();
    int64_t best_row = -1;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int q = half * 32 + (lane & 31);
      const int64_t row = bj + 32 * (q >> 4) + 8 * ((q & 15) >> 2) + (q & 3);
      const bool ok = row < c_hi && row < p.V;
      const f32x16 c = block_logits(ok ? p.W + row * p.H : nullptr, p.X + tj * p.H, p.H, lane);
      // Every column is the same token: read the rows from column 0's lanes
      // (lanes 0 and 32 hold rows 8(r/4) + r%4 and 8(r/4) + 4 + r%4).
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int qi = half * 32 + i;
        const int64_t ri = bj + 32 * (qi >> 4) + 8 * ((qi & 15) >> 2) + (qi & 3);
        const bool oki = ri < c_hi && ri < p.V && (lane & 31) == 0;
        if (oki && c[r] > best) {
          best = c[r];
          best_row = ri;
        }
      }
    }
    // Reduce over lanes 0 and 32 (the others hold no candidate), then hand
    // the result to every lane.
    const float ob = __shfl(best, lane ^ 32);
    const int orow = __shfl((int)best_row, lane ^ 32);
    if (ob > best || (ob == best && orow >= 0 && (best_row < 0 || orow < best_row))) {
      best = ob;
      best_row = orow;
    }
    best = __shfl(best, 0);
    best_row = __shfl((int)best_row, 0);
    // The token's own lane holds its row terms.  The label's entry, when it
    // is the dominant one, has been taken above.
    if (lane == jt && best_row >= 0 && best > zthr && best_row != wrow) {
      float pr, d;
      const float val = grad_value<kCapped, kGen>(best, off, gsc, c1, p.eps_over_v, k2, c2, l2a, pr, d);
      p.dom_col[tj] = (int32_t)(best_row + p.key_offset);
      p.dom_coef[tj] = val - vinf;
      const int64_t g = g_offset(tj, best_row - c_lo, p.n_vtiles);
      p.G[g] = vinf_bits;
      if (p.G_lo) p.G_lo[g] = vinf_lo;
    }
  }
}

}  // namespace

hipError_t launch_exact_entries(const ExactParams& p, hipStream_t stream) {
  if (p.N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((p.N + kExactRows - 1) / kExactRows));
  const bool capped = p.softcap > 0.0f, gen = p.gs != nullptr;
  if (capped && gen) hipLaunchKernelGGL((exact_entries_kernel<true, true>), grid, dim3(64), 0, stream, p);
  else if (capped) hipLaunchKernelGGL((exact_entries_kernel<true, false>), grid, dim3(64), 0, stream, p);
  else if (gen) hipLaunchKernelGGL((exact_entries_kernel<false, true>), grid, dim3(64), 0, stream, p);
  else hipLaunchKernelGGL((exact_entries_kernel<false, false>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace lce
