// Device-side building blocks shared by the gfx950 kernels of liblce.
//
// Tiles: one workgroup of 256 threads (4 waves of 64) computes a 256 x 256
// fp32 tile C = A · Bᵀ over a K range, 64 K-values per pipeline step.  Each
// wave owns a 128 x 128 quarter as 4 x 4 blocks of the 32x32x16 bf16 MFMA.
// Operands are staged through LDS.  A K-major stage holds its 64 K values as
// two K-halves of 32; in each half a tile row is 64 bytes (four 16-byte
// chunks), so that one 16-byte LDS read gives a lane its 8-element MFMA
// fragment.  The chunks of a row are XOR-swizzled by the row index to keep
// the fragment reads and the tile writes free of bank conflicts.
//
// MFMA lane layout (v_mfma_f32_32x32x16_bf16, checked on gfx950):
//   A fragment: lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]
//   B fragment: lane l holds B[8*(l/32) .. +7][l % 32]   (i.e. Bᵀ row l % 32)
//   C/D:        lane l, element r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kTile = 256;      // output tile edge (both M and N)
constexpr int kBK = 64;         // K values per pipeline step
constexpr int kWaveTile = 128;  // each wave: 128 x 128
constexpr int kMI = 4;          // 32x32 MFMA blocks per wave along M
constexpr int kNI = 4;          // ... along N
constexpr int kStageElems = kTile * kBK;      // bf16 elements per operand per stage
constexpr int kXcds = 8;                      // MI355X: 8 XCDs ...
constexpr int kCusPerXcd = 32;                // ... of 32 compute units

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh(x) = 1 - 2 / (exp(2x) + 1); saturates correctly at +-inf.
// `two_log2e_over_c` folds x = z / c and the base change into one multiply.
__device__ __forceinline__ float tanh_of_scaled(float z, float two_log2e_over_c) {
  float e = exp2_fast(z * two_log2e_over_c);
  return 1.0f - 2.0f * rcp_fast(e + 1.0f);
}

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two floats -> packed bf16 pair (lo, hi), round to nearest even; gfx950 does
// this in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// K-major LDS stage of one operand: K-half h (K values 32h .. 32h+31) at
// element h·kHalfElems, 256 rows of 32 values (64 bytes).  The pipeline
// refills a half as soon as its last slice has been read, so the loads of a
// step spread over the whole step instead of crowding into one quarter of it.
// Swizzle: 16-byte chunk c of row r sits at c ^ ((r / 4) % 4); 16 consecutive
// rows reading one logical chunk then hit 16 distinct 16-byte bank groups
// (rows r and r + 4k differ in the swizzle, rows r .. r+3 in the 64-byte slot).
constexpr int kHalfK = kBK / 2;               // K values per half
constexpr int kHalfElems = kTile * kHalfK;    // bf16 elements per half (16 KiB)
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ int lds_off(int half, int row, int chunk) {
  return half * kHalfElems + row * kHalfK + ((chunk ^ swz(row)) << 3);
}

// ----------------------------------------------------------------------------
// Buffer descriptors.  A descriptor covers `bytes` bytes from `base` (capped
// at 2^31 − 1); the hardware range check turns every access at an offset at
// or beyond that size into a zero read or a dropped write.  All of an
// access's offset is carried in the VGPR operand so the check sees it.
// kOutOfRange plus any in-tile offset (< 2^30) stays out of range.
// ----------------------------------------------------------------------------
constexpr uint32_t kBufferConfig = 0x00020000u;  // raw 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;    // offset that always reads 0

// Compiler-visible form, for the epilogue loads and stores of fp32 tiles.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kBufferConfig);
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}
__device__ __forceinline__ void buffer_store_f32(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)voff, 0, 0);
}

// ----------------------------------------------------------------------------
// Direct-to-LDS loads, issued through inline asm.
//
// buffer_load_dwordx4 ... lds writes each lane's 16 bytes to LDS at
// M0 + 16·lane instead of to registers.  Issued through the compiler's builtin,
// the compiler tracks these writes and, for LDS reads it cannot prove
// disjoint (the transposing reads below), inserts a full vmcnt(0) wait after
// every load, which serialises the pipeline.  Issued as asm, the compiler
// tracks none of them; the pipeline itself guarantees visibility: every
// stage is read only after an explicit vmcnt(0) and a workgroup barrier.
// (Compiler-inserted vmcnt waits for its own loads stay correct: loads
// complete in order, so extra outstanding loads only make them stricter.)
// M0 is written here and nowhere else in these kernels.
// ----------------------------------------------------------------------------
typedef u32x4 rsrc_t;

// Raw buffer descriptor: base, stride 0, size in bytes (capped at 2^31 − 1),
// raw 32-bit data format.
__device__ __forceinline__ rsrc_t make_rsrc_raw(const uint16_t* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  r[3] = kBufferConfig;
  return r;
}

__device__ __forceinline__ void dtl16(const rsrc_t& rsrc, const void __attribute__((address_space(3)))* lds,
                                      uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc)
               : "memory");
}

// ----------------------------------------------------------------------------
// Direct-to-LDS K-major loader (buffer_load_dwordx4 ... lds).  One wave
// instruction fills a 1 KiB block of one K-half: tile rows 16b .. 16b+15,
// lane l writing bytes [16·l, 16·l+16) of it (checked on gfx950: out-of-range
// lanes write zeros), i.e. row 16b + l/4 at physical chunk l % 4, so the lane
// fetches logical chunk (l % 4) ^ swz(row) of the half.  swz(16b + l/4) =
// (l/16) % 4 for every block, so a lane's K offset is the same in every block
// it fills.  A step is 8 instructions per wave: q = 0..3 fill half 0 (blocks
// 4q + wave), q = 4..7 half 1 (blocks 4(q − 4) + wave).
// ----------------------------------------------------------------------------
#define LCE_LDS __attribute__((address_space(3)))

template <bool kTail>
struct DtlKMajorTile {
  rsrc_t rsrc;
  uint32_t voff;      // byte offset of this lane's chunk in half 0, block `wave`
  uint32_t row_step;  // bytes between blocks 4j + wave and 4(j+1) + wave (64 rows)
  int32_t kchunk;     // this lane's K offset inside a half
  int32_t wave;       // wave index, wave-uniform (kept in an SGPR)
  int64_t k_total;

  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int64_t row0,
                                       int64_t rows_total, int64_t k_total_, int tid) {
    rsrc = make_rsrc_raw(base + row0 * ld, (rows_total - row0) * ld * 2);
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = wave * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    kchunk = c * 8;
    k_total = k_total_;
    voff = (uint32_t)(row * ld * 2 + c * 16);
    row_step = (uint32_t)(64 * ld * 2);
  }
  // Per-step state: the lane's byte offsets of its chunk in half 0 and half 1
  // of the 64-deep K block at k0 (kOutOfRange: a zero fill, for chunks past
  // k_total when kTail, and for steps past the end of the K range).
  // `row_bytes` moves the step to tile rows further on inside the same
  // descriptor (the next tile of a sweep).
  struct Step {
    uint32_t b0, b1;
  };
  __device__ __forceinline__ Step prepare(int64_t k0, uint32_t row_bytes = 0) const {
    uint32_t b0 = voff + row_bytes + (uint32_t)(k0 * 2), b1 = b0 + kHalfK * 2;
    if (kTail) {
      b0 = (k0 + kchunk < k_total) ? b0 : kOutOfRange;
      b1 = (k0 + kHalfK + kchunk < k_total) ? b1 : kOutOfRange;
    }
    return Step{b0, b1};
  }
  __device__ __forceinline__ Step null_step() const { return Step{kOutOfRange, kOutOfRange}; }
  // Enqueue load q (0..7) of the step into `stage`: asynchronous, complete
  // once this wave's vmcnt has drained past it.  Without kTail, k_total must
  // be a multiple of 64 so every chunk is in range.  kOutOfRange plus the
  // block offset (< 2^30) stays out of range.
  __device__ __forceinline__ void issue(const Step& st, LCE_LDS uint16_t* stage, int q) const {
    const int h = q >> 2, j = q & 3;
    dtl16(rsrc, stage + h * kHalfElems + (j * 4 + wave) * 512, (h ? st.b1 : st.b0) + j * row_step);
  }
  __device__ __forceinline__ void load(LCE_LDS uint16_t* stage, int64_t k0) const {
    const Step st = prepare(k0);
#pragma unroll
    for (int q = 0; q < 8; ++q) issue(st, stage, q);
  }
};

// Direct-to-LDS MN-major loader: the tile's contiguous dimension m runs along
// memory rows of length ld (element (m, k) at base[k·ld + m]).  LDS holds the
// tile as 64 rows (one per k) of 256 m values = 512 B, its 16-byte chunks
// XOR-swizzled by 4·(k % 4) so that the transposing fragment reads below hit
// 16 distinct 16-byte bank groups.  One wave instruction fills two LDS rows
// (1 KiB, lane l -> row l/32, physical chunk l % 32); blocks 4i + wave.
// K rows at or beyond k_total read as zero (the descriptor ends there);
// columns past the end of a memory row only reach output columns that are
// never stored.
__device__ __forceinline__ int mn_off(int k, int m) {
  return k * 256 + ((((m >> 3) ^ ((k & 3) << 2))) << 3) + (m & 7);
}

struct DtlMNMajorTile {
  const uint16_t* base;
  int64_t ld, k_total;
  uint32_t voff, row_step;
  int32_t wave;

  __device__ __forceinline__ void init(const uint16_t* base_, int64_t ld_, int64_t col0,
                                       int64_t /*cols_total*/, int64_t k_total_, int tid) {
    base = base_;
    ld = ld_;
    k_total = k_total_;
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = 2 * wave + (lane >> 5);  // + 8i for block 4i + wave; row % 4 fixed
    const int c = (lane & 31) ^ ((row & 3) << 2);
    voff = (uint32_t)(row * ld * 2 + (col0 + c * 8) * 2);
    row_step = (uint32_t)(8 * ld * 2);
  }
  // Per-step state: a descriptor starting at K row k0 and ending at k_total.
  struct Step {
    rsrc_t rsrc;
  };
  __device__ __forceinline__ Step prepare(int64_t k0) const {
    return Step{make_rsrc_raw(base + k0 * ld, (k_total - k0) * ld * 2)};
  }
  __device__ __forceinline__ Step null_step() const { return Step{make_rsrc_raw(base, 0)}; }
  // Load q fills K rows 2·wave + 8q and 2·wave + 8q + 1, so q = 0..3 cover
  // K-half 0 (rows 0..31) and q = 4..7 K-half 1.
  __device__ __forceinline__ void issue(const Step& st, LCE_LDS uint16_t* stage, int i) const {
    dtl16(st.rsrc, stage + wave * 512 + i * 2048, voff + i * row_step);
  }
  __device__ __forceinline__ void load(LCE_LDS uint16_t* stage, int64_t k0) const {
    const Step st = prepare(k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue(st, stage, i);
  }
};

// ----------------------------------------------------------------------------
// Blocked layout of the logit-gradient chunk G.  For token tile t and
// chunk-local vocabulary tile j, the 256 x 256 block sits at element
// (t·nvt + j)·65536 and is stored as 4 sub-blocks of 64 vocabulary columns,
// each 256 token rows of 64 contiguous values:
//   G[tok][v] at (t·nvt + j)·65536 + (v%256 / 64)·16384 + (tok%256)·64 + v%64.
// Every pipeline step of both contractions then reads contiguous memory: a
// 64-column K step of dX (tokens x vocabulary) is one 32 KiB sub-block, a
// 64-row K step of dW (vocabulary x tokens) four 8 KiB pieces.  Rows of the
// last token tile past N are stored as zeros by the writer.
// ----------------------------------------------------------------------------
constexpr int64_t kGBlockElems = (int64_t)kTile * kTile;  // one 256 x 256 block
constexpr int64_t kGSubElems = (int64_t)kTile * kBK;      // one 256 x 64 sub-block

// K-major reader of blocked G for the dX contraction: rows are the tokens of
// one token tile, K the chunk's vocabulary.  init(G, nvt, tok0, ...): the
// second argument is the chunk's count of vocabulary tiles.  Same LDS image
// as DtlKMajorTile; in memory, K-half h of token row r of K step k0 is the
// 64 bytes at sub-block k0 / 64, row r, column 32h.
struct DtlKMajorBlockedG {
  rsrc_t rsrc;
  uint32_t voff, row_step;
  int32_t wave;
  __device__ __forceinline__ void init(const uint16_t* base, int64_t nvt, int64_t row0,
                                       int64_t /*rows_total*/, int64_t /*k_total*/, int tid) {
    rsrc = make_rsrc_raw(base + (row0 / kTile) * nvt * kGBlockElems, nvt * kGBlockElems * 2);
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = wave * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    voff = (uint32_t)(row * kBK * 2 + c * 16);
    row_step = (uint32_t)(64 * kBK * 2);
  }
  struct Step {
    uint32_t b0, b1;
  };
  // K step k0 (a multiple of 64) is sub-block k0 / 64 of the token tile.
  __device__ __forceinline__ Step prepare(int64_t k0) const {
    const uint32_t b0 = voff + (uint32_t)(k0 / kBK) * (uint32_t)(kGSubElems * 2);
    return Step{b0, b0 + kHalfK * 2};
  }
  __device__ __forceinline__ Step null_step() const { return Step{kOutOfRange, kOutOfRange}; }
  __device__ __forceinline__ void issue(const Step& st, LCE_LDS uint16_t* stage, int q) const {
    const int h = q >> 2, j = q & 3;
    dtl16(rsrc, stage + h * kHalfElems + (j * 4 + wave) * 512, (h ? st.b1 : st.b0) + j * row_step);
  }
  __device__ __forceinline__ void load(LCE_LDS uint16_t* stage, int64_t k0) const {
    const Step st = prepare(k0);
#pragma unroll
    for (int q = 0; q < 8; ++q) issue(st, stage, q);
  }
};

// MN-major reader of blocked G for the dW contraction: M is the chunk-local
// vocabulary tile starting at col0 (a multiple of 256), K the tokens.  Same
// lane-to-LDS mapping as DtlMNMajorTile (LDS row k, swizzled 16-byte chunk
// c of 8 columns); only the global address differs.  init(G, nvt, col0, ...).
struct DtlMNMajorBlockedG {
  const uint16_t* base;
  int64_t nvt, vt;
  uint32_t voff, row_step;
  int32_t wave;
  __device__ __forceinline__ void init(const uint16_t* base_, int64_t nvt_, int64_t col0,
                                       int64_t /*cols_total*/, int64_t /*k_total*/, int tid) {
    base = base_;
    nvt = nvt_;
    vt = col0 / kTile;
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = 2 * wave + (lane >> 5);  // + 8i for block 4i + wave
    const int c = (lane & 31) ^ ((row & 3) << 2);
    voff = (uint32_t)((c >> 3) * kGSubElems * 2 + row * kBK * 2 + (c & 7) * 16);
    row_step = (uint32_t)(8 * kBK * 2);
  }
  struct Step {
    rsrc_t rsrc;
  };
  // K step k0 (64 tokens of token tile k0 / 256): a descriptor from the
  // step's first row to the end of the block.
  __device__ __forceinline__ Step prepare(int64_t k0) const {
    const int64_t blk = ((k0 / kTile) * nvt + vt) * kGBlockElems;
    const int64_t first = (k0 % kTile) * kBK;
    return Step{make_rsrc_raw(base + blk + first, (kGBlockElems - first) * 2)};
  }
  __device__ __forceinline__ Step null_step() const { return Step{make_rsrc_raw(base, 0)}; }
  __device__ __forceinline__ void issue(const Step& st, LCE_LDS uint16_t* stage, int i) const {
    dtl16(st.rsrc, stage + wave * 512 + i * 2048, voff + i * row_step);
  }
  __device__ __forceinline__ void load(LCE_LDS uint16_t* stage, int64_t k0) const {
    const Step st = prepare(k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue(st, stage, i);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// MFMA fragment of tile rows mbase .. mbase+31, K slice t (16 deep).
// K-major LDS: one 16-byte read (slice t lies in half t / 2, chunks
// 2·(t % 2) and 2·(t % 2) + 1 for the two lane halves).  MN-major LDS: two ds_read_b64_tr_b16.  That
// instruction works on groups of 16 lanes: lane k supplies 4 consecutive
// elements P_k and lane i receives P_{4j + i/4}[i % 4], j = 0..3 (checked on
// gfx950).  Pointing lane k' at k-row (k0 + k'/4), columns m0 + 4(k' % 4)
// therefore hands lane i the 4 consecutive k of column m0 + i.
template <bool kMN>
__device__ __forceinline__ bf16x8 frag_read(const LCE_LDS uint16_t* s, int mbase, int t, int lane) {
  if (!kMN) {
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const LCE_LDS u32x4*>(
                    s + lds_off(t >> 1, mbase + (lane & 31), ((t & 1) << 1) | (lane >> 5))));
  } else {
    const int g = lane >> 4, kk = lane & 15;
    const int m = mbase + 16 * (g & 1) + 4 * (kk & 3);
    const int k0 = t * 16 + 8 * (g >> 1) + (kk >> 2);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCE_LDS s16x4*)(s + mn_off(k0, m)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LCE_LDS s16x4*)(s + mn_off(k0 + 4, m)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]).
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
constexpr int kWaitVm16 = (1 << 14) | (7 << 4) | (15 << 8);       // vmcnt <= 16
constexpr int kWaitVm20 = (1 << 14) | 4 | (7 << 4) | (15 << 8);   // vmcnt <= 20
constexpr int kWaitVm8 = 8 | (7 << 4) | (15 << 8);                 // vmcnt <= 8
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (3 << 14);

// Workgroup barrier without the memory fence __syncthreads() carries (that
// fence would drain every outstanding direct-to-LDS load).  Callers wait for
// the loads that must be visible with an explicit vmcnt first; the empty asm
// statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// MFMA operand fragments of one 16-deep K slice for a wave's 128 x 128 quarter.
struct Frag {
  bf16x8 a[kMI], b[kNI];
};

template <bool kAmn, bool kBmn>
__device__ __forceinline__ void read_frag(Frag& f, const LCE_LDS uint16_t* sA,
                                          const LCE_LDS uint16_t* sB, int wm, int wn, int lane,
                                          int t) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi) f.a[mi] = frag_read<kAmn>(sA, wm * kWaveTile + mi * 32, t, lane);
#pragma unroll
  for (int ni = 0; ni < kNI; ++ni) f.b[ni] = frag_read<kBmn>(sB, wn * kWaveTile + ni * 32, t, lane);
}

#define LCE_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Fragment piece p (0..7) of K slice t: A rows for p < 4, B rows otherwise.
template <bool kAmn, bool kBmn>
__device__ __forceinline__ void read_piece(Frag& f, const LCE_LDS uint16_t* sA,
                                           const LCE_LDS uint16_t* sB, int wm, int wn, int lane,
                                           int t, int p) {
  if (p < kMI)
    f.a[p] = frag_read<kAmn>(sA, wm * kWaveTile + p * 32, t, lane);
  else
    f.b[p - kMI] = frag_read<kBmn>(sB, wn * kWaveTile + (p - kMI) * 32, t, lane);
}

// Cross-tile prefetch state of a persistent sweep over A tiles that share one
// B tile (the forward and the logit-gradient kernels walk the vocabulary
// tiles of one token tile).  The load stream of a tile runs on into the next
// tile: its last two steps issue that tile's steps 0 and 1, so those loads
// are in flight during the caller's epilogue and the next tile starts
// without a pipeline fill.
struct Sweep {
  int par = 0;             // stage index holding step 0 of the current tile
  bool preloaded = false;  // steps 0 and 1 of the current tile are in flight
};

// One section of a pipeline step: the 16 MFMAs of fragment set `fm` (one
// 16-deep K slice), the 8 fragment pieces of K slice t of stage (rA, rB) into
// `fr`, and (kLoad) 4 loads of one operand's K-half h into `dst`, loads
// 4h .. 4h+3 of the step state `st`.  The reads go with the first 8 MFMAs, so
// they land well before the next section multiplies them; the loads go with
// every fourth MFMA.  Each group is fenced so the compiler keeps the
// interleave.  kZeroC: the MFMAs start from zero instead of acc (the first K
// slice of a tile).
template <bool kAmn, bool kBmn, bool kLoad, class L, bool kZeroC = false>
__device__ __forceinline__ void pipe_section(const Frag& fm, Frag& fr, const LCE_LDS uint16_t* rA,
                                             const LCE_LDS uint16_t* rB, int t, const L& ld,
                                             const typename L::Step& st, LCE_LDS uint16_t* dst,
                                             int h, int wm, int wn, int lane,
                                             f32x16 (&acc)[kMI][kNI]) {
  const f32x16 zero = {};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mi = i >> 2, ni = i & 3;
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fm.a[mi], fm.b[ni], kZeroC ? zero : acc[mi][ni],
                                                          0, 0, 0);
    if (i < 8) read_piece<kAmn, kBmn>(fr, rA, rB, wm, wn, lane, t, i);
    if (kLoad && (i & 3) == 3) ld.issue(st, dst, 4 * h + (i >> 2));
    LCE_SCHED_FENCE();
  }
}

// Section boundary: this wave's loads older than its last kNewer (16, 8 or
// 0: the loads issued after the awaited group) have landed and its LDS reads
// are done; then the same for every wave.
template <int kNewer>
__device__ __forceinline__ void pipe_barrier() {
  __builtin_amdgcn_s_waitcnt(kNewer >= 16 ? kWaitVm16 : (kNewer >= 8 ? kWaitVm8 : kWaitVm0));
  lds_barrier();
}

// One 256 x 256 tile C += A·Bᵀ over the K range [k_begin, k_end) (at least
// one 64-deep step), each operand K-major (kAmn/kBmn false) or MN-major
// (true), through a two-stage direct-to-LDS pipeline.  LDS: 128 KiB (stage s
// of A at smem + s·kStageElems, of B at smem + (2 + s)·kStageElems).  For a
// K-major operand `row0/rows` are its tile rows; for an MN-major one they are
// its column offset / column count.
//
// A step is four sections of 16 MFMAs, one per 16-deep K slice; the
// fragments of a slice are read from LDS in the section before the one that
// multiplies them.  With S the stage of step k (halves h0 = slices 0-1,
// h1 = slices 2-3) and each step's loads in four groups (h0 of A, h0 of B,
// h1 of A, h1 of B):
//   A(k): MFMA slice 0, read slice 1 (S.h0), load step k+1 h1 of B
//   barrier: every wave has read S.h0; step k's h1 has landed
//   B(k): MFMA slice 1, read slice 2 (S.h1), load step k+2 h0 of A into S.h0
//   C(k): MFMA slice 2, read slice 3 (S.h1), load step k+2 h0 of B into S.h0
//   barrier: every wave has read S.h1; step k+1's h0 has landed
//   E(k): MFMA slice 3, read slice 0 of step k+1, load step k+2 h1 of A into S.h1
// Every section thus carries 8 fragment reads (two LDS reads each for an
// MN-major operand) and 4 loads per wave, and a load has about four sections
// to land.  Each wait counts the loads issued after the awaited group: 16
// inside the K range.  A sweep keeps that count to the end (its last tile
// loads zeros for the steps past the range); a single tile peels its last
// two steps, which load nothing and wait for 8 or 0.  The last step still
// reads the next step's first slice, unused.
//
// kSweep (K-major operands only, k_begin = 0): the tile overwrites acc
// (C = A·Bᵀ; its first K slice starts from zero) and `sw` carries the prefetch
// state; when next_a_row0 >= 0 and the tile has at least two steps, the steps
// past the K range are steps 0 and 1 of the next A tile (rows next_a_row0 >
// a_row0, within a_rows; same B), so the next call finds them in flight.  kWaitAll: the caller issues other
// memory operations between two tiles, so a preloaded tile waits for all of
// them (vmcnt 0).
// Without a next tile every load has landed when the tile returns; after a
// sweep the caller waits for vmcnt 0 before reusing the LDS.
//
// kABlk: A is the blocked gradient chunk (DtlKMajorBlockedG / DtlMNMajorBlockedG);
// `lda` is then the chunk's count of vocabulary tiles.
template <bool kAmn, bool kBmn, bool kTail, bool kSweep = false, bool kWaitAll = false,
          bool kABlk = false>
__device__ __forceinline__ void gemm_tile(const uint16_t* A, int64_t lda, int64_t a_row0,
                                          int64_t a_rows, const uint16_t* B, int64_t ldb,
                                          int64_t b_row0, int64_t b_rows, int64_t k_begin,
                                          int64_t k_end, int64_t k_total, LCE_LDS uint16_t* smem,
                                          f32x16 (&acc)[kMI][kNI], Sweep* sw = nullptr,
                                          int64_t next_a_row0 = -1) {
  typedef typename std::conditional<
      kABlk, typename std::conditional<kAmn, DtlMNMajorBlockedG, DtlKMajorBlockedG>::type,
      typename std::conditional<kAmn, DtlMNMajorTile, DtlKMajorTile<kTail>>::type>::type LA;
  typedef typename std::conditional<kBmn, DtlMNMajorTile, DtlKMajorTile<kTail>>::type LB;
  typedef typename LA::Step StA;
  typedef typename LB::Step StB;
  static_assert(!kSweep || (!kAmn && !kBmn), "the sweep prefetch handles K-major operands");
  static_assert(!kSweep || !kABlk, "the sweep prefetch reads row-major operands");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nsteps = (int)((k_end - k_begin + kBK - 1) / kBK);
  const int par = kSweep ? sw->par : 0;
  // The stream runs on into the next tile only when a tile has at least two
  // steps: a step loads step k+2 two sections ahead, so with one step per tile
  // (K <= 64) that would skip the next tile's step 0 and load its (absent)
  // step 1 instead.  A one-step tile starts the next one with its own prologue.
  const bool prefetch = kSweep && next_a_row0 >= 0 && nsteps >= 2;
  LA la;
  LB lb;
  la.init(A, lda, a_row0, a_rows, k_total, tid);
  lb.init(B, ldb, b_row0, b_rows, k_total, tid);
  // Sweep: the next A tile lies next_a_row0 − a_row0 rows further on, inside
  // the descriptor of this one (it ends at a_rows).
  const uint32_t next_bytes = prefetch ? (uint32_t)((next_a_row0 - a_row0) * lda * 2) : 0u;
  // Stage of stream step s: A at smem + ((par + s) % 2)·kStageElems.
  auto stA = [&](int s) { return smem + ((par ^ s) & 1) * kStageElems; };
  auto stB = [&](int s) { return smem + (2 + ((par ^ s) & 1)) * kStageElems; };
  // Loader state of stream step s: this tile's steps, then (sweep with a next
  // tile) that tile's steps 0 and 1.  Past those, a sweep loads zeros into
  // stages no longer read; a single tile loads nothing (its tail steps).
  auto stepA = [&](int s) -> StA {
    if (s < nsteps) return la.prepare(k_begin + (int64_t)s * kBK);
    if constexpr (kSweep) {
      if (prefetch) return la.prepare((int64_t)(s - nsteps) * kBK, next_bytes);
    }
    return la.null_step();
  };
  auto stepB = [&](int s) -> StB {
    if (s < nsteps) return lb.prepare(k_begin + (int64_t)s * kBK);
    if constexpr (kSweep) {
      if (prefetch) return lb.prepare((int64_t)(s - nsteps) * kBK);
    }
    return lb.null_step();
  };
  if (kSweep && sw->preloaded) {
    // Steps 0 and 1 (28 loads per wave, as below) were issued by the previous tile.
    if (kWaitAll) __builtin_amdgcn_s_waitcnt(kWaitVm0);
    else __builtin_amdgcn_s_waitcnt(kWaitVm20);
  } else {
    lds_barrier();  // every wave is done with the LDS of the previous tile
    // Steps 0 and 1 in steady-state order, except step 1's h1 of B, which
    // section A of step 0 issues.
    const StA a0 = stepA(0), a1 = stepA(1);
    const StB b0 = stepB(0), b1 = stepB(1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < 4; ++q) la.issue(a0, stA(0), 4 * h + q);
#pragma unroll
      for (int q = 0; q < 4; ++q) lb.issue(b0, stB(0), 4 * h + q);
    }
    if (kSweep || nsteps > 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) la.issue(a1, stA(1), q);
#pragma unroll
      for (int q = 0; q < 4; ++q) lb.issue(b1, stB(1), q);
#pragma unroll
      for (int q = 4; q < 8; ++q) la.issue(a1, stA(1), q);
      __builtin_amdgcn_s_waitcnt(kWaitVm20);   // step 0's h0 has landed
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
    }
  }
  lds_barrier();
  Frag f0, f1, f2, f3;
  read_frag<kAmn, kBmn>(f0, stA(0), stB(0), wm, wn, lane, 0);
  LCE_SCHED_FENCE();
  StB bnext = stepB(1);  // step k+1 of B, for section A of step k
  // Step k; L1 / L2: steps k+1 / k+2 are loaded (compile-time flags, so no
  // branch sits between the MFMAs).
  auto step = [&](int k, auto L1, auto L2, auto Z) {
    constexpr bool l1 = decltype(L1)::value, l2 = decltype(L2)::value, z = decltype(Z)::value;
    LCE_LDS uint16_t* ca = stA(k);
    LCE_LDS uint16_t* cb = stB(k);
    LCE_LDS uint16_t* na = stA(k + 1);
    LCE_LDS uint16_t* nb = stB(k + 1);
    const StA a2 = stepA(k + 2);
    const StB b2 = stepB(k + 2);
    pipe_section<kAmn, kBmn, l1, LB, z>(f0, f1, ca, cb, 1, lb, bnext, nb, 1, wm, wn, lane, acc);
    pipe_barrier<l1 ? 16 : 0>();
    pipe_section<kAmn, kBmn, l2>(f1, f2, ca, cb, 2, la, a2, ca, 0, wm, wn, lane, acc);
    pipe_section<kAmn, kBmn, l2>(f2, f3, ca, cb, 3, lb, b2, cb, 0, wm, wn, lane, acc);
    pipe_barrier<(l1 ? 8 : 0) + (l2 ? 8 : 0)>();
    pipe_section<kAmn, kBmn, l2>(f3, f0, na, nb, 0, la, a2, ca, 1, wm, wn, lane, acc);
    bnext = b2;
  };
  const std::true_type yes{};
  const std::false_type no{};
  int k = 0;
  if constexpr (kSweep) {
    // The stream runs on into the next tile's steps 0 and 1, or, after the
    // last tile, loads zeros into stages no longer read (one code path for
    // every tile keeps the accumulators in place).  Step 0 starts the
    // accumulators from zero.
    step(k++, yes, yes, yes);
    for (; k < nsteps; ++k) step(k, yes, yes, no);
  } else {
    for (; k + 2 < nsteps; ++k) step(k, yes, yes, no);
    if (k + 1 < nsteps) step(k++, yes, no, no);
    step(k, no, no, no);
  }
  if (kSweep) {
    sw->par = (par + nsteps) & 1;  // stage of the next tile's step 0
    sw->preloaded = prefetch;
  }
}

// Map a logical workgroup id of a (token tile, split) grid so that each XCD
// (a contiguous range of nwg/8 logical ids after xcd_remap) covers a tt x ss
// block of token tiles x vocabulary splits: per pipeline step the XCD then
// touches tt distinct X blocks and ss distinct W blocks.  tt == 0 keeps the
// plain order (token tile fastest).
__device__ __forceinline__ void grid_tile(int g, int T, int tt, int ss, int& ti, int& split) {
  if (tt == 0) {
    ti = g % T;
    split = g / T;
    return;
  }
  const int per = tt * ss, x = g / per, local = g % per, ngt = T / tt;
  ti = (x % ngt) * tt + local % tt;
  split = (x / ngt) * ss + local / tt;
}

// Oversubscribed (token tile, split) grid, in rounds of kXcds·kCusPerXcd
// workgroups: round r covers token tiles [r·rt, (r + 1)·rt) with every split
// (rt·S = kXcds·kCusPerXcd), and within the round the workgroups of XCD x
// (hardware id % 8) take a (rt / 8) x S block of it.  Workgroups start in id
// order, so the ones resident together form about one round, and each XCD's
// block shares its X and W blocks in L2.  In a partly filled last round (the
// host launches full rounds only) ti would pass the last token tile; the
// caller skips such a workgroup.
__device__ __forceinline__ void round_tile(int b, int rt, int& ti, int& split) {
  const int per_round = kXcds * kCusPerXcd;
  const int r = b / per_round, q = b - r * per_round;
  const int x = q % kXcds, local = q / kXcds, tt = rt / kXcds;
  ti = r * rt + x * tt + local % tt;
  split = local / tt;
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[kMI][kNI]) {
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
}

// Row (within the 256-row tile) of accumulator element r of block mi for `lane`.
__device__ __forceinline__ int acc_row(int wm, int mi, int r, int lane) {
  return wm * kWaveTile + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
// Compile-time part of acc_row: acc_row = acc_row_lane(wm, lane) + acc_row_const(mi, r).
__device__ __forceinline__ int acc_row_lane(int wm, int lane) { return wm * kWaveTile + 4 * (lane >> 5); }
__device__ __forceinline__ constexpr int acc_row_const(int mi, int r) { return mi * 32 + 8 * (r >> 2) + (r & 3); }
// Column (within the 256-column tile) of block ni for `lane`.
__device__ __forceinline__ int acc_col(int wn, int ni, int lane) {
  return wn * kWaveTile + ni * 32 + (lane & 31);
}

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Map the
// hardware id to a logical id so that each XCD receives a contiguous range of
// logical ids; neighbouring logical tiles then share operands in one L2.
__device__ __forceinline__ int xcd_remap(int b, int nwg) {
  const int per = nwg >> 3;
  if (b >= per * 8) return b;
  return (b & 7) * per + (b >> 3);
}

// Value of one logit-gradient entry from its logit z (the same arithmetic in
// every kernel that forms it).  Plain form (kGen false): G = p·d, `off`
// folding the row class in (−inf for ignored rows, so G = 0; NaN for rows with
// a bad label).  General form: G = gsc·(c1·p − eps_v)·d with the row's scale
// gsc (0 ignored, NaN bad) and Z-loss factor c1.  p is the softmax value and d
// the softcap derivative (1 without).  Without softcap off = −lse2; with
// softcap c, r = 1/(2^(z·k2) + 1) gives tanh = 1 − 2r, off = c2 − lse2 + 2,
// pr4 = 2^(off − 2·c2·r) = 4p, and d = 4r(1 − r).  (k2 = 2a·log2 e / c,
// c2 = c·log2 e, l2a = a·log2 e, lse2 = LSE·log2 e.)
template <bool kCapped, bool kGen>
__device__ __forceinline__ float grad_value(float z, float off, float gsc, float c1, float eps_v,
                                            float k2, float c2, float l2a, float& pr, float& d) {
  if (kCapped) {
    const float rr = rcp_fast(exp2_fast(z * k2) + 1.0f);
    const float pr4 = exp2_fast(fmaf(-2.0f * c2, rr, off));
    const float dq = fmaf(-rr, rr, rr);
    pr = 0.25f * pr4;
    d = 4.0f * dq;
    return kGen ? gsc * fmaf(c1, pr4, -4.0f * eps_v) * dq : pr4 * dq;
  } else {
    pr = exp2_fast(fmaf(z, l2a, off));
    d = 1.0f;
    return kGen ? gsc * fmaf(c1, pr, -eps_v) : pr;
  }
}

// Softmax threshold of a dominant entry: 1/2 + 2^-10, so that two entries of
// one row can never both lie above it.
constexpr float kDominantP = 0.5009765625f;

// The raw logit above which an entry's softmax exceeds kDominantP, for a row
// with exponent offset `off` as in grad_value (+inf when `live` is false:
// rows without a gradient have no dominant entry).
template <bool kCapped>
__device__ __forceinline__ float dominance_threshold(bool live, float off, float k2, float c2,
                                                     float l2a) {
  float zthr = __builtin_inff();
  if (!live) return zthr;
  const float log2tau = __builtin_log2f(kDominantP);
  if (kCapped) {
    // p > τ  <=>  off − 2·c2·r > 2 + log2 τ  <=>  r < R  <=>  z > log2(1/R − 1)/k2.
    const float R = (off - 2.0f - log2tau) / (2.0f * c2);
    if (R > 0.0f && R < 1.0f) zthr = log2f(1.0f / R - 1.0f) / k2;
  } else {
    zthr = (log2tau - off) / l2a;
  }
  return zthr;
}

// Index checks of the debug build (build.py --debug-checks): LCE_DCHECK(c)
// is c, and prints the failing check, so that `if (LCE_DCHECK(i < n)) use(i)`
// skips the access it guards; the product build compiles it to true.
#ifdef LCE_DEBUG_CHECKS
__device__ __forceinline__ bool lce_dcheck(bool ok, const char* what, const char* file, int line) {
  if (!ok) printf("lce check failed: %s (%s:%d)\n", what, file, line);
  return ok;
}
#define LCE_DCHECK(cond) lce_dcheck((cond), #cond, __FILE__, __LINE__)
#else
#define LCE_DCHECK(cond) true
#endif

// Row classes written by the row-preparation kernels.
enum RowState : int32_t { kRowIgnored = 0, kRowValid = 1, kRowBad = 2 };

}  // namespace lce
