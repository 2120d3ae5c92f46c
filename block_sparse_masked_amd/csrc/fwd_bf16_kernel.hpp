// Kernel of the bf16 forward, shared by the contiguous-KV and paged-KV
// translation units (fwd_bf16.hip, fwd_bf16_paged.hip).
//
// Block-sparse attention forward, bf16 inputs, fp32 accumulation, gfx950.
//
// The forward of page "tensorplay.nn.attention API" (BlockMask "Details"
// item 1: reduce along KV over each query row-tile's tile lists; item 2:
// mask_mod only on partial tiles) computed tile by tile with an online
// softmax, so the score matrix is never materialised (page "Attention
// Backends", section "Why care about Attention Kernels?"; page
// "FlagAttention", tiling with recomputation). GQA: query head h reads KV head
// h / (Hq / Hkv) (page "FlagAttention", section "Operator overview").
//
// Work decomposition: one workgroup of 4 waves per (b, h, 128-row query
// tile); wave w owns query rows [32w, 32w + 32). Two workgroups share a CU
// (three at head dim 64), so each SIMD runs two (three) waves and one wave's
// softmax (vector ALUs) overlaps another's matrix products. Both products use v_mfma_f32_32x32x16_bf16:
//   S^T = K . Q^T    (A = K rows from LDS, B = Q^T held in registers)
//   O^T += V^T . P^T (A = V^T read transposed from LDS, B = P^T in registers)
// The MFMA result's lane index is the query column, so each lane holds the
// scores of one query row (half of a step's keys); the row max needs one
// exchange with lane ^ 32, the P^T operand is the converted score registers
// and the O^T accumulator is rescaled per lane.
//
// Short query tiles (Q_LEN <= 64, mask broadcast over heads) give each query
// head one or two waves and fill the workgroup with 4 or 2 heads of one KV
// group, which then share the K/V stream. With one wave per head and at most
// 16 query rows, both products use v_mfma_f32_16x16x32_bf16 instead (the
// 16-row step: lane l holds query l % 16, lane group l / 16 a quarter of
// each 16-key block), so no matrix work goes to empty rows.
//
// MFMA 32x32 result layout: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32. An operand register slot t of
// lane l holds k = 8*(l/32) + t for both A and B, so the key order inside the
// P.V contraction follows the S result layout directly.
//
// KV is walked in steps of 64 keys at D = 64 and 128 (a step's K or V block
// is 8 or 16 KiB) and 32 keys at D = 256, each BlockMask tile in 128 / NK
// steps.
// K and V of step g + 1 are loaded straight from global memory into LDS
// (double-buffered) while step g computes; one barrier per step.
// Full tiles take a path with no mask code. The running max is applied
// lazily: O and the row sums are rescaled only when a row's max grows by more
// than 8 (log2 units), which skips most rescales; any reference point gives
// the same normalised sums in exact arithmetic. In rounded arithmetic the
// row's largest probability can then be up to 2^8 instead of exactly 1, and
// its rounding to the input type would go straight into O; so for the
// score-mod kinds O is divided by the fp32 sum of the rounded probabilities
// (the values the P.V product multiplies), and LSE uses the sum of the
// unrounded ones, which the plain kinds also divide O by (kRoundedSum).
#pragma once

#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "fwd_common.hpp"
#include "fwd_plan.hpp"
#include "launch.hpp"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The 16-bit input element: bf16 (F16 = false) or fp16. Both have the same
// register and LDS layouts and a 32x32x16 MFMA with fp32 accumulation; P is
// rounded to the input type for the P.V product.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// sum8: c + the 8 rounded probabilities of one P operand register set, in
// fp32 (four two-element dot products with (1, 1)): the row sum of exactly
// the values the P.V product multiplies.
template <bool F16>
struct Elem {
  using T = __bf16;
  using V8 = bf16x8;
  using V4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sum8(V8 p, float c) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), one, c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), one, c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), one, c, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), one, c, false);
  }
};
template <>
struct Elem<true> {
  using T = _Float16;
  using V8 = f16x8;
  using V4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sum8(V8 p, float c) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    c = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 0, 1), one, c, false);
    c = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 2, 3), one, c, false);
    c = __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 4, 5), one, c, false);
    return __builtin_amdgcn_fdot2(__builtin_shufflevector(p, p, 6, 7), one, c, false);
  }
};
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int kWavesPerHead = 4;  // 4 x 32 query rows = one 128-row query tile
constexpr float kRescaleSlack = 8.0f;  // exp2 units: p <= 256 between rescales
constexpr int kStepBytes = 16384;      // one K (or V) step block in LDS (D >= 128)
// Step block bytes per head dim. D = 64 takes 8 KiB blocks (64-key steps):
// the kernel then needs at most 166 VGPRs and 32 KiB of step buffers, so
// three workgroups share a CU (three waves per SIMD), which keeps the matrix
// cores busier while the vector units bound the head dim's softmax.
template <int D>
constexpr int step_bytes() { return D == 64 ? 8192 : kStepBytes; }
template <int D>
constexpr int wg_per_cu() { return D > 128 ? 1 : (D == 64 ? 3 : 2); }

// internal score kind: plain scaled score with the scale applied before the
// row max (needed when scale < 0; SCORE_NONE folds the scale into exp2)
constexpr int SCORE_SCALED = 4;

template <int D>
struct Geom {
  static constexpr int NK = step_bytes<D>() / (2 * D);  // keys per step
  static constexpr int SPT = kBlock / NK;          // steps per BlockMask tile
  static constexpr int NB = NK / 32;               // 32-key blocks per step
  static constexpr int NE = NB * 16;               // scores per lane per step
  static constexpr int PKS = NK / 16;              // P.V k-steps per step
  static constexpr int KS = D / 16;                // S k-steps
  static constexpr int DB = D / 32;                // O d-blocks
};

struct FwdArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  long long sq0, sq1, sq2, sk0, sk1, sv0, sv1, so0, so1, so2;
  int sk2, sv2;  // key-row strides (elements, < 2^22)
  int B, Hq, Hkv, G, Q_LEN, KV_LEN;
  int xcd_round;  // > 0: items per schedule round, remapped so KV groups share an XCD
  // waves per query head (one-head workgroups): 4 covers a 128-row query
  // tile; 2 or 1 (Q_LEN <= 64 or <= 32, mask broadcast over heads) gives the
  // other waves further heads of the same KV group, so short query tiles do
  // not leave most MFMA rows idle and the group's K/V are read once
  int wph;
  int doc_len;
  MaskParams mp;
  float c_scale, c_cap, cap2;
  const float* slopes;
  BlockMaskView bm;
  // split-KV: each item's tile list is cut into `splits` contiguous slices,
  // one workgroup each, writing fp32 partial results (O normalised by its
  // slice's row sum, and the slice's LSE) that a combine pass merges
  int splits;     // 1: no split, O and LSE written directly
  float* part_o;  // [splits][B][Hq][Q_LEN][D]
  float* part_lse;  // [splits][B][Hq][Q_LEN]
  // paged KV (page_table != nullptr): k and v are caches of num_pages pages
  // of page_size key rows each (sk0 / sv0 are page strides); key j of batch
  // b is row j % page_size of page page_table[b * pt_stride + j / page_size].
  // page_size is a multiple of 128, so a BlockMask tile lies in one page.
  const int* page_table;
  int page_size, pt_stride, num_pages;
  // optional fp32 copy of O, contiguous [B][Hq][Q_LEN][D] (unsplit calls):
  // the backward's row sums Delta = dO . O are then one pass over it
  float* o32;
};

// 16-byte chunk swizzle of a K block [NK][D] in LDS: the 16 rows a 16-lane
// phase of a fragment read touches land in distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  if constexpr (D >= 128) {
    return col ^ (row & 15);
  } else {
    return col ^ ((row >> 1) & 7);
  }
}

// V block swizzle for the transposed reads: two 16-lane groups read the same
// 4 consecutive rows at chunk pairs c, c+1 and c+2, c+3 (c = 4 * d-block).
// XOR-ing with 4*(row%4) (D = 128: 16 chunks per 256-byte row) or with
// 4*((row/2)%2) (D = 64: 8 chunks per 128-byte row, two rows per bank sweep)
// gives those 16 half-chunk pairs distinct banks.
template <int D>
__device__ __forceinline__ int swz_v(int row, int col) {
  if constexpr (D >= 128) {
    return col ^ ((row & 3) << 2);
  } else {
    return col ^ (((row >> 1) & 1) << 2);
  }
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(unsigned long long)(__attribute__((address_space(3))) const void*)p;
}

// Buffer resource for raw loads: 64-bit base, no stride, `bytes` in range
// (loads past it read as zero). Built from wave-uniform values.
__device__ __forceinline__ i32x4 make_rsrc(unsigned long long base, unsigned bytes) {
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)base);
  r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(base >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Direct global->LDS loads (16 and 4 bytes per lane). Written as asm with
// no register results: the LDS they fill is a buffer no instruction reads
// until after the explicit vmcnt(0) + barrier that ends the step, so the
// compiler need not (and does not) wait for them. No memory clobber: the asm
// stays ordered against the barriers and waits (all have side effects),
// while the LDS reads of the other buffer may be scheduled around it. Each
// load takes the CU's vector-memory path for a few cycles, so the step
// spreads them between its matrix instructions.
// The load's LDS address is M0, passed as an operand bound to M0 (the
// compiler writes it and knows it is used); the address is wave-uniform by
// construction and readfirstlane states that to the compiler. The
// compiler's hazard recognizer does not look inside inline asm, so the
// block keeps the CDNA wait states itself: an LDS DMA needs one wait state
// after a scalar write of M0 (without it the load can take the previous M0,
// i.e. land on the previous load's LDS slot), and a vector memory
// instruction five after a vector instruction wrote one of its scalar
// operands (the resource words come from readfirstlane): s_nop 4 gives five.
#define FA_LDS_DMA(op) "s_nop 4\n\t" op " %0, %1, 0 offen lds"
__device__ __forceinline__ void dma16(i32x4 rsrc, unsigned lds, int voff) {
  asm volatile(FA_LDS_DMA("buffer_load_dwordx4")
               : : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds)));
}
__device__ __forceinline__ void dma4(i32x4 rsrc, unsigned lds, int voff) {
  asm volatile(FA_LDS_DMA("buffer_load_dword")
               : : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds)));
}
#undef FA_LDS_DMA

// Loads of one [NK][D] step block of K or V. Each wave-wide load fills one
// contiguous KiB of LDS (lane l writes bytes [16 l, 16 l + 16)), so each lane
// fetches the global chunk whose swizzled home is that slot; its byte offset
// from the block's first row is fixed and computed once. Per step only the
// resource moves; its range ends with key KV_LEN - 1 (see range_bytes), and
// the scores of rows past it are masked: a tile crossing KV_LEN takes the
// masked path.
template <int D, bool IS_V, int WAVES>
struct BlockLoader {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWS_PER_KB = 1024 / (2 * D);
  static constexpr int KB_PER_WAVE = step_bytes<D>() / 1024 / WAVES;
  static constexpr int NK = Geom<D>::NK;
  int voff[KB_PER_WAVE];
  unsigned long long base;  // byte address of key row 0 of this (b, kv head)
  unsigned row_bytes;
  unsigned lds0;            // LDS byte address of this wave's first KiB, buffer 0

  __device__ void init(const u16* g, int stride, int wave, int lane, const u16* lds_buf0) {
    base = reinterpret_cast<unsigned long long>(g);
    row_bytes = 2u * (unsigned)stride;
    const int r_in = lane / CPR;
    const int pch = lane % CPR;
#pragma unroll
    for (int i = 0; i < KB_PER_WAVE; ++i) {
      const int row = (wave * KB_PER_WAVE + i) * ROWS_PER_KB + r_in;
      const int col = IS_V ? swz_v<D>(row, pch) : swz<D>(row, pch);
      voff[i] = row * (int)row_bytes + col * 16;
    }
    lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_buf0) + wave * KB_PER_WAVE * 1024);
  }

  // loads of keys [kv0, kv0 + NK) into buffer `buf` (its LDS is lds0 + buf * 2 * kStepBytes
  // when the two buffers of K (or V) are laid out [buf][K|V])
  // The range ends with the last valid row's data, not at rows * row_bytes,
  // so a row stride below the row length (0 for keys broadcast along the
  // sequence) still reads every valid row; rows past it read as zero when
  // the stride is the row length or more, else other valid rows (their
  // scores are masked either way).
  __device__ __forceinline__ unsigned range_bytes(int rows) const {
    return rows > 0 ? (unsigned)(rows - 1) * row_bytes + 2u * D : 0u;
  }
  __device__ __forceinline__ i32x4 plan(int kv0, int kv_len) const {
    const int rows = min(kv_len - kv0, NK);
    return make_rsrc(base + (unsigned long long)kv0 * row_bytes, range_bytes(rows));
  }
  __device__ __forceinline__ void issue_one(i32x4 rsrc, unsigned lds_buf, int i) const {
    dma16(rsrc, lds_buf + 1024 * i, voff[i]);
  }
  __device__ __forceinline__ void issue(int kv0, int kv_len, unsigned lds_buf) const {
    const int rows = min(kv_len - kv0, NK);
    const i32x4 rsrc = make_rsrc(base + (unsigned long long)kv0 * row_bytes, range_bytes(rows));
#pragma unroll
    for (int i = 0; i < KB_PER_WAVE; ++i) dma16(rsrc, lds_buf + 1024 * i, voff[i]);
  }
};

__device__ __forceinline__ void wait_loads_and_sync() {
  // vmcnt(0), expcnt/lgkmcnt unconstrained, then the workgroup barrier
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

template <bool F16>
__device__ __forceinline__ typename Elem<F16>::V8 as_v8(uint4 u) {
  typename Elem<F16>::V8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// Per-lane context of one work item, including the LDS element offsets of
// this lane's fragments. The swizzles only XOR row bits that are the same
// for every block / k-step a lane reads, so one offset per K k-step and one
// per V d-block suffice; the rest of each address is a compile-time constant.
template <int D>
struct Lane {
  int lane, l32, hh, vg, vi;
  int q, qc;
  // the wave's query rows (32-row layout, wave-uniform): qc of its first
  // and last lane
  int qw_lo, qw_hi;
  float slope2;
  int dq;            // document id of this lane's query row (document mask)
  int kofs[D / 16];  // K fragment (row l32 of block 0, k-step ks)
  int vofs[D / 32];  // V transposed-read piece (k-step 0, half 0, d-block db)
  // 16-row layout (v_mfma_f32_16x16x32): query lane % 16, key group lane / 16
  int c16, g4;
  int kofs16[D / 32];  // K fragment (row c16 of block 0, k-step ks: d 32 ks + 8 g4)
  int vofs16[D / 16];  // V transposed-read piece (rows 4 g4 + c16 / 4, d-block db)

  __device__ void init_offsets() {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kofs[ks] = l32 * D + swz<D>(l32, 2 * ks + hh) * 8;
    // + 16*ks + 8*half: multiples of 4 leave row % 4 and (row / 2) % 2 alone
    const int row = 4 * hh + (vi >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = 32 * db + 16 * vg + 4 * (vi & 3);
      vofs[db] = row * D + swz_v<D>(row, d >> 3) * 8 + (d & 7);
    }
  }

  // 16-row layout: the swizzles only XOR row bits that adding 16 (K) or
  // 16 / 32 (V) rows leaves alone, so one offset per k-step and d-block
  __device__ void init_offsets16() {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) kofs16[ks] = c16 * D + swz<D>(c16, 4 * ks + g4) * 8;
    const int row = 4 * g4 + (c16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d = 16 * db + 4 * (c16 & 3);
      vofs16[db] = row * D + swz_v<D>(row, d >> 3) * 8 + (d & 7);
    }
  }
};

// Row max across the two lanes that hold one query row (lane, lane ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                   false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// V^T operand fragment for P.V MFMA (k-step ks, d-block db): lane row
// d = 32*db + lane%32, slot t <-> key 16*ks + 8*(t/4) + 4*hh + t%4 (the key
// order of pf), read from the row-major V block with two transposing reads:
// in each 16-lane group lane j supplies the 8-byte piece (row j/4, columns
// 4*(j%4)..+3) of a 4-key x 16-d block and receives column j of that block.
template <int D, bool F16>
__device__ __forceinline__ typename Elem<F16>::V8 v_frag(const u16* sV, const Lane<D>& ln, int ks,
                                                         int db) {
  typename Elem<F16>::V4 part[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const u16* src = sV + ln.vofs[db] + (16 * ks + 8 * ht) * D;
    const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(src));
    __builtin_memcpy(&part[ht], &raw, 8);
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// K operand fragment for S MFMA (k-step ks, key block blk): rows
// 32*blk + lane%32 keep row % 16 (and (row/2) % 8), so one offset per k-step.
template <int D, bool F16>
__device__ __forceinline__ typename Elem<F16>::V8 k_frag(const u16* sK, const Lane<D>& ln, int ks,
                                                         int blk) {
  return as_v8<F16>(*reinterpret_cast<const uint4*>(sK + ln.kofs[ks] + 32 * blk * D));
}

// Key offset (within the step, without 4*hh) of result register r of block blk.
__device__ __forceinline__ constexpr int key_off(int blk, int r) {
  return 32 * blk + 8 * (r >> 2) + (r & 3);
}

// Per-step mask limits: key offset c (see key_off) is allowed when c <= hi,
// and for the sliding window also c > win_lo or c < sink_hi; for documents
// the key's id (LDS) must equal the query row's.
struct MaskLimits {
  int hi, win_lo, sink_hi;
  int tlo[kMaxTerms], thi[kMaxTerms];  // COMPOSITE: allowed offsets of each term
};

// base: the key the lane's offsets count from (kv0 + 4*hh in the 32-row
// layout, kv0 + 4*g4 in the 16-row one).
template <int D, int MASK>
__device__ __forceinline__ MaskLimits mask_limits(int base, const FwdArgs& a, const Lane<D>& ln) {
  MaskLimits m;
  m.hi = a.KV_LEN - 1 - base;
  if constexpr (MASK == MASK_PREFIX_LM) m.hi = min(m.hi, max(ln.qc, a.mp.prefix - 1) - base);
  else if constexpr (MASK != MASK_NOOP && MASK != MASK_COMPOSITE) m.hi = min(m.hi, ln.qc - base);
  m.win_lo = ln.qc - base - a.mp.window;
  m.sink_hi = a.mp.sinks - base;
  if constexpr (MASK == MASK_COMPOSITE) {
#pragma unroll
    for (int t = 0; t < kMaxTerms; ++t) {
      int lo = 1, hi = 0;  // unused terms allow nothing
      if (t < a.mp.nterms) {
        term_interval(a.mp.terms[t], ln.qc, a.mp, lo, hi);
        hi = min(hi, a.KV_LEN - 1) - base;
        lo -= base;
      }
      m.tlo[t] = lo;
      m.thi[t] = hi;
    }
  }
  return m;
}

// Whether any key of a step can be allowed for this lane's query row, from
// the step's mask limits over the offsets [0, nk) (a superset of the lane's
// keys; document ids are not consulted, so a document test never rules a
// step out).
template <int MASK>
__device__ __forceinline__ bool step_may_attend(const MaskLimits& ml, int nk) {
  const int top = min(ml.hi, nk - 1);
  bool any = top >= 0;
  if constexpr (MASK == MASK_SLIDING_SINK) {
    const bool in_window = max(ml.win_lo + 1, 0) <= top;
    const bool in_sinks = min(ml.sink_hi - 1, top) >= 0;
    any = any & (in_window | in_sinks);
  }
  if constexpr (MASK == MASK_COMPOSITE) {
    bool t_any = false;
#pragma unroll
    for (int t = 0; t < kMaxTerms; ++t) t_any = t_any | (max(ml.tlo[t], 0) <= min(ml.thi[t], top));
    any = any & t_any;
  }
  return any;
}

// Mask test of one 32-key block of a step, keys [k0, k0 + 31], for every
// row of the wave at once (interval masks: causal, sliding window with
// sinks, PrefixLM): 0 when every key is allowed for every row, 1 when none
// is, 2 when the elements must be tested one by one. Decided from the wave's
// row range, conservatively (a block that is neither all allowed nor all
// masked for certain is tested per element); wave-uniform.
template <int D, int MASK>
__device__ __forceinline__ int block_mode(int k0, const FwdArgs& a, const Lane<D>& ln) {
  const int k1 = k0 + 31;
  bool all = k1 < a.KV_LEN;
  bool none = k0 >= a.KV_LEN;
  if constexpr (MASK == MASK_CAUSAL) {
    all = all & (k1 <= ln.qw_lo);
    none = none | (k0 > ln.qw_hi);
  } else if constexpr (MASK == MASK_SLIDING_SINK) {
    all = all & (k1 <= ln.qw_lo) & ((ln.qw_hi - k0 < a.mp.window) | (k1 < a.mp.sinks));
    none = none | (k0 > ln.qw_hi) | ((ln.qw_lo - k1 >= a.mp.window) & (k0 >= a.mp.sinks));
  } else if constexpr (MASK == MASK_PREFIX_LM) {
    all = all & ((k1 < a.mp.prefix) | (k1 <= ln.qw_lo));
    none = none | ((k0 >= a.mp.prefix) & (k0 > ln.qw_hi));
  }
  return __builtin_amdgcn_readfirstlane(all ? 0 : (none ? 1 : 2));
}

// Score-mod kinds (ALiBi, softcap, both) form each logit relative to the
// reference max in use before the step, z = y - m_old, from one per-step,
// per-lane constant
//   zbase = [cap2] + [slope2 * (first key of the lane - q)] - m_old
// and the register's compile-time key offset c:
//   softcap:  z = cap2 * (1 - 2 / (exp(2 s / cap) + 1)) + ... = fma(r, -2 cap2, t)
//   ALiBi:    t = fma(slope2, c, zbase), z = fma(s, scale, t) without softcap
// so the bias costs one FMA per score and exp2(z) needs no subtraction (a
// step that raises the reference shifts its z once, in the rare rescale).
template <int SCORE>
constexpr bool kRelLogit =
    SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP || SCORE == SCORE_SOFTCAP_ALIBI;

// O's divisor. With the lazy reference a row's largest probability can be up
// to 2^8 and is then not exact in the input type; where it dominates the row,
// its rounding would reach O by up to 2^-9 of |V|. The score-mod kinds (whose
// biases and caps make such rows common) divide by the fp32 sum of the
// rounded probabilities P.V multiplies, so the weights sum to one whatever
// the rounding; the plain kinds divide by the fp32 sum of the probabilities
// (the LSE's sum), which saves a quarter of an instruction per score.
template <int SCORE>
constexpr bool kRoundedSum = kRelLogit<SCORE>;

template <int SCORE>
__device__ __forceinline__ float rel_logit(float x, float c, float zbase, const FwdArgs& a,
                                           float slope2) {
  constexpr bool kSoft = SCORE == SCORE_SOFTCAP || SCORE == SCORE_SOFTCAP_ALIBI;
  constexpr bool kAlibi = SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI;
  const float t = kAlibi ? fmaf(slope2, c, zbase) : zbase;
  if constexpr (kSoft) {
    const float e = fast_exp2(x * a.c_cap);
    return fmaf(fast_rcp(e + 1.0f), -2.0f * a.cap2, t);
  } else {
    return fmaf(x, a.c_scale, t);
  }
}

template <int SCORE>
__device__ __forceinline__ float rel_logit_base(float m_old, int key0_minus_q, const FwdArgs& a,
                                                float slope2) {
  float z = -m_old;
  if constexpr (SCORE == SCORE_SOFTCAP || SCORE == SCORE_SOFTCAP_ALIBI) z += a.cap2;
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
    z = fmaf(slope2, (float)key0_minus_q, z);
  return z;
}

// Mask test of one score of a partial tile (32-row layout).
template <int D, int MASK>
__device__ __forceinline__ bool elem_allowed(int blk, int r, const MaskLimits& ml,
                                             const int* step_doc, const FwdArgs& a,
                                             const Lane<D>& ln) {
  // conditions combined with & and |, not && and ||: every operand is
  // safe to evaluate (the document ids of the step are in LDS), and
  // short-circuit forms turned each element's test into a branch
  const int c = key_off(blk, r);
  bool ok = c <= ml.hi;
  if constexpr (MASK == MASK_SLIDING_SINK) ok = ok & ((c > ml.win_lo) | (c < ml.sink_hi));
  if constexpr (MASK == MASK_DOCUMENT) ok = ok & (step_doc[c + 4 * ln.hh] == ln.dq);
  if constexpr (MASK == MASK_COMPOSITE) {
    bool any = false;
    const bool same_doc = step_doc[c + 4 * ln.hh] == ln.dq;  // ids in LDS (composite)
#pragma unroll
    for (int t = 0; t < kMaxTerms; ++t) {
      bool in = (c >= ml.tlo[t]) & (c <= ml.thi[t]);
      if (a.mp.terms[t] & PRIM_DOCUMENT) in = in & same_doc;
      any = any | in;
    }
    ok = ok & any;
  }
  return ok;
}

// Logit of one score: y = score_mod(x) in base-2 units (raw x for
// SCORE_NONE, scaled later; z = y - m_old for the score-mod kinds), -inf
// where masked on partial tiles.
template <int D, int MASK, int SCORE, bool MASKED>
__device__ __forceinline__ float elem_logit(float x, int blk, int r, float zbase,
                                            const MaskLimits& ml, const int* step_doc,
                                            const FwdArgs& a, const Lane<D>& ln) {
  float y = x;
  if constexpr (SCORE == SCORE_SCALED) {
    y = x * a.c_scale;
  } else if constexpr (kRelLogit<SCORE>) {
    y = rel_logit<SCORE>(x, (float)key_off(blk, r), zbase, a, ln.slope2);
  }
  if constexpr (MASKED) y = elem_allowed<D, MASK>(blk, r, ml, step_doc, a, ln) ? y : -INFINITY;
  return y;
}

// One KV step: S = K . Q^T, online softmax, O += V . P. `dma(i)` issues the
// i-th of the NDMA loads of the next step (called between S products).
template <int D, int MASK, int SCORE, bool MASKED, int NDMA, bool F16, typename DMA>
__device__ __forceinline__ void step(f32x16 (&o)[D / 32], float& m_ref, float& l, float& lp,
                                     const typename Elem<F16>::V8 (&qf)[D / 16], const u16* sK,
                                     const u16* sV,
                                     int kv0, const int* step_doc, const FwdArgs& a,
                                     const Lane<D>& ln, DMA&& dma) {
  using G = Geom<D>;
  f32x16 s[G::NB];
#pragma unroll
  for (int b = 0; b < G::NB; ++b) s[b] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks)
#pragma unroll
    for (int b = 0; b < G::NB; ++b)
    {
      const auto kf = k_frag<D, F16>(sK, ln, ks, b);
      s[b] = Elem<F16>::mfma(kf, qf[ks], s[b]);
      // the next step's loads, spread over the S products
      constexpr int NS = G::KS * G::NB;
      static_assert(NS % NDMA == 0, "loads spread evenly");
      const int i = ks * G::NB + b;
      if (i % (NS / NDMA) == 0) dma(i / (NS / NDMA));
    }

  const MaskLimits ml = mask_limits<D, MASK>(kv0 + 4 * ln.hh, a, ln);
  constexpr bool kRel = kRelLogit<SCORE>;
  const float m_old = (m_ref == -INFINITY) ? 0.0f : m_ref;
  const float zbase =
      kRel ? rel_logit_base<SCORE>(m_old, kv0 + 4 * ln.hh - ln.q, a, ln.slope2) : 0.0f;
  // logits; on partial tiles a 32-key block is tested per element only
  // when the wave's rows do not all agree on it (a wave-uniform branch)
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < G::NB; ++b) {
    // (only for the interval masks without a score mod: the score-mod
    // kinds' logits need more registers and the branches made the compiler
    // spill; a document block would need its key ids read and compared,
    // which cost more than the tests it saved)
    constexpr bool kElide = MASKED && !kRel &&
        (MASK == MASK_CAUSAL || MASK == MASK_SLIDING_SINK || MASK == MASK_PREFIX_LM);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      s[b][r] = elem_logit<D, MASK, SCORE, MASKED && !kElide>(s[b][r], b, r, zbase, ml, step_doc,
                                                              a, ln);
    if constexpr (kElide) {
      const int mode = block_mode<D, MASK>(kv0 + 32 * b, a, ln);
      if (mode == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] = -INFINITY;
      } else if (mode == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[b][r] = elem_allowed<D, MASK>(b, r, ml, step_doc, a, ln) ? s[b][r] : -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
  }
  mx = pair_max(mx);
  if constexpr (SCORE == SCORE_NONE) mx *= a.c_scale;  // c_scale > 0 here

  // lazy rescale (a real branch: rare); relative logits compare against the
  // slack directly (any finite logit when there is no reference yet)
  const float thr = kRel ? ((m_ref == -INFINITY) ? -INFINITY : kRescaleSlack)
                         : m_ref + kRescaleSlack;
  if (__any(mx > thr)) {
    asm volatile("");
    const float m_new = fmaxf(m_ref, kRel ? mx + m_old : mx);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_ref - m_new);
    l *= alpha;
    lp *= alpha;
#pragma unroll
    for (int i = 0; i < G::DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    m_ref = m_new;
    if constexpr (kRel) {
      const float delta = ((m_new == -INFINITY) ? 0.0f : m_new) - m_old;
#pragma unroll
      for (int b = 0; b < G::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[b][r] -= delta;
    }
  }
  const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;

  typename Elem<F16>::V8 pf[G::PKS];
  float rs = 0.0f;
#pragma unroll
  for (int e = 0; e < G::NE; ++e) {
    const float y = s[e >> 4][e & 15];
    float p;
    if constexpr (SCORE == SCORE_NONE) {
      p = fast_exp2(fmaf(y, a.c_scale, -m_use));
    } else if constexpr (kRel) {
      p = fast_exp2(y);
    } else {
      p = fast_exp2(y - m_use);
    }
    rs += p;
    pf[e >> 3][e & 7] = (typename Elem<F16>::T)p;
  }
  l += rs;
  // the rounded sum only where a score mod can make one probability
  // dominate a row with a value the input type does not hold exactly
  if constexpr (kRoundedSum<SCORE>) {
#pragma unroll
    for (int ks = 0; ks < G::PKS; ++ks) lp = Elem<F16>::sum8(pf[ks], lp);
  }

#pragma unroll
  for (int ks = 0; ks < G::PKS; ++ks)
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
      const auto vf = v_frag<D, F16>(sV, ln, ks, db);
      o[db] = Elem<F16>::mfma(vf, pf[ks], o[db]);
    }
}

// ---------------------------------------------------------------------------
// 16-row step (query tiles of at most 16 rows, such as decode): per wave one
// query head of 16 rows, v_mfma_f32_16x16x32 for both products, so no MFMA
// rows are idle. Result layout: register r of lane l holds row 4*(l/16) + r,
// column l%16; operand slot t of lane l holds k = 8*(l/16) + t. S^T = K.Q^T
// puts keys 16*blk + 4*g4 + r of the step on the lane's registers (query
// c16); in the P.V contraction slot t of pair j stands for key
// 32*j + 16*(t/4) + 4*g4 + t%4, and V^T is read in that order.
// ---------------------------------------------------------------------------
template <int D, bool F16>
__device__ __forceinline__ typename Elem<F16>::V8 k_frag16(const u16* sK, const Lane<D>& ln,
                                                           int ks, int blk) {
  return as_v8<F16>(*reinterpret_cast<const uint4*>(sK + ln.kofs16[ks] + 16 * blk * D));
}

template <int D, bool F16>
__device__ __forceinline__ typename Elem<F16>::V8 v_frag16(const u16* sV, const Lane<D>& ln, int j,
                                                           int db) {
  typename Elem<F16>::V4 part[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const u16* src = sV + ln.vofs16[db] + (32 * j + 16 * ht) * D;
    const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(src));
    __builtin_memcpy(&part[ht], &raw, 8);
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(typename Elem<F16>::V8 a, typename Elem<F16>::V8 b,
                                        f32x4 c) {
  if constexpr (F16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Logit of score r of 16-key block blk (key kv0 + 16*blk + 4*g4 + r).
template <int D, int MASK, int SCORE, bool MASKED>
__device__ __forceinline__ float elem_logit16(float x, int blk, int r, float zbase,
                                              const MaskLimits& ml, const int* step_doc,
                                              const FwdArgs& a, const Lane<D>& ln) {
  float y = x;
  const int c = 16 * blk + r;  // offset within the step, without 4*g4
  if constexpr (SCORE == SCORE_SCALED) {
    y = x * a.c_scale;
  } else if constexpr (kRelLogit<SCORE>) {
    y = rel_logit<SCORE>(x, (float)c, zbase, a, ln.slope2);
  }
  if constexpr (MASKED) {
    bool ok = c <= ml.hi;
    if constexpr (MASK == MASK_SLIDING_SINK) ok = ok & ((c > ml.win_lo) | (c < ml.sink_hi));
    if constexpr (MASK == MASK_DOCUMENT) ok = ok & (step_doc[c + 4 * ln.g4] == ln.dq);
    if constexpr (MASK == MASK_COMPOSITE) {
      bool any = false;
      const bool same_doc = step_doc[c + 4 * ln.g4] == ln.dq;  // ids in LDS (composite)
#pragma unroll
      for (int t = 0; t < kMaxTerms; ++t) {
        bool in = (c >= ml.tlo[t]) & (c <= ml.thi[t]);
        if (a.mp.terms[t] & PRIM_DOCUMENT) in = in & same_doc;
        any = any | in;
      }
      ok = ok & any;
    }
    y = ok ? y : -INFINITY;
  }
  return y;
}

template <int D, int MASK, int SCORE, bool MASKED, int NDMA, bool F16, typename DMA>
__device__ __forceinline__ void step16(f32x4 (&o)[D / 16], float& m_ref, float& l, float& lp,
                                       const typename Elem<F16>::V8 (&qf)[D / 16], const u16* sK,
                                       const u16* sV, int kv0, const int* step_doc,
                                       const FwdArgs& a, const Lane<D>& ln, DMA&& dma) {
  constexpr int NK = Geom<D>::NK;
  constexpr int NB = NK / 16;  // 16-key blocks per step
  constexpr int KS = D / 32;   // S k-steps
  constexpr int DB = D / 16;   // O d-blocks
  f32x4 s[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) s[b] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      s[b] = mfma16<F16>(k_frag16<D, F16>(sK, ln, ks, b), qf[ks], s[b]);
      constexpr int NS = KS * NB;
      static_assert(NS % NDMA == 0, "loads spread evenly");
      const int i = ks * NB + b;
      if (i % (NS / NDMA) == 0) dma(i / (NS / NDMA));
    }

  // the mask limits relative to key kv0 + 4*g4
  const MaskLimits ml = mask_limits<D, MASK>(kv0 + 4 * ln.g4, a, ln);
  constexpr bool kRel = kRelLogit<SCORE>;
  const float m_old = (m_ref == -INFINITY) ? 0.0f : m_ref;
  const float zbase =
      kRel ? rel_logit_base<SCORE>(m_old, kv0 + 4 * ln.g4 - ln.q, a, ln.slope2) : 0.0f;
  float mx = -INFINITY;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[b][r] = elem_logit16<D, MASK, SCORE, MASKED>(s[b][r], b, r, zbase, ml, step_doc, a, ln);
      mx = fmaxf(mx, s[b][r]);
    }
  // a query's keys are spread over lanes c16, c16 + 16, c16 + 32, c16 + 48
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if constexpr (SCORE == SCORE_NONE) mx *= a.c_scale;  // c_scale > 0 here

  const float thr = kRel ? ((m_ref == -INFINITY) ? -INFINITY : kRescaleSlack)
                         : m_ref + kRescaleSlack;
  if (__any(mx > thr)) {
    asm volatile("");
    const float m_new = fmaxf(m_ref, kRel ? mx + m_old : mx);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_ref - m_new);
    l *= alpha;
    lp *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[i][r] *= alpha;
    m_ref = m_new;
    if constexpr (kRel) {
      const float delta = ((m_new == -INFINITY) ? 0.0f : m_new) - m_old;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[b][r] -= delta;
    }
  }
  const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;

  typename Elem<F16>::V8 pf[NB / 2];
  float rs = 0.0f;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float y = s[b][r];
      float p;
      if constexpr (SCORE == SCORE_NONE) {
        p = fast_exp2(fmaf(y, a.c_scale, -m_use));
      } else if constexpr (kRel) {
        p = fast_exp2(y);
      } else {
        p = fast_exp2(y - m_use);
      }
      rs += p;
      pf[b >> 1][4 * (b & 1) + r] = (typename Elem<F16>::T)p;
    }
  l += rs;  // this lane's keys; the four lanes of a query are summed at the end
  if constexpr (kRoundedSum<SCORE>) {
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) lp = Elem<F16>::sum8(pf[j], lp);
  }

#pragma unroll
  for (int j = 0; j < NB / 2; ++j)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      o[db] = mfma16<F16>(v_frag16<D, F16>(sV, ln, j, db), pf[j], o[db]);
}

// Four waves per workgroup, two workgroups per CU (two waves per SIMD);
// three at D = 64.
// D = 256 holds 128 accumulator and 64 Q registers per lane: one workgroup
// per CU, with the accumulators in the matrix-core registers.
// R16: the 16-row step for query tiles of at most 16 rows (one query head
// per wave, 4 heads of a KV group per workgroup).
template <int D, int MASK, int SCORE, bool PAGED, bool F16, bool R16>
__global__ __launch_bounds__(64 * kWavesPerHead, wg_per_cu<D>()) void
fwd_bf16_kernel(FwdArgs a) {
  using E = Elem<F16>;
  using G = Geom<D>;
  constexpr int WAVES = kWavesPerHead;
  constexpr int THREADS = 64 * WAVES;
  constexpr int NK = G::NK;
  constexpr int SPT = G::SPT;
  constexpr int STEP_ELEMS = step_bytes<D>() / 2;
  // LDS: K and V step blocks double-buffered (separate arrays, so the
  // compiler can tell the buffer being filled from the one being read and does
  // not wait for in-flight loads before LDS reads), two document-id buffers,
  // and the item's tile list (NKB ints, dynamic)
  __shared__ __attribute__((aligned(16))) u16 sK0[STEP_ELEMS];
  __shared__ __attribute__((aligned(16))) u16 sK1[STEP_ELEMS];
  __shared__ __attribute__((aligned(16))) u16 sV0[STEP_ELEMS];
  __shared__ __attribute__((aligned(16))) u16 sV1[STEP_ELEMS];
  // document ids are fetched 64 at a time (one wave-wide 4-byte load), so a
  // buffer holds at least 64 even when a step has fewer keys (D = 256)
  constexpr int DOC_STRIDE = NK > 64 ? NK : 64;
  __shared__ __attribute__((aligned(16))) int docbuf[mask_uses_doc(MASK) ? 2 * DOC_STRIDE : 1];
  extern __shared__ __attribute__((aligned(16))) int tlist[];

  // dispatch order -> item; rounds of equal tile count are remapped so the
  // heads sharing a KV head run on one XCD (workgroups go round-robin to XCDs)
  int x = blockIdx.x;
  int split = 0;
  if (a.splits > 1) {
    split = x % a.splits;
    x /= a.splits;
  }
  // BLOCK_SIZE = mk * 128: a tile row holds mk 128-row query tiles (one item
  // each) and a listed tile mk 128-key tiles (walked one after another)
  const int mk = a.bm.BS / kBlock, mq = a.bm.QBS / kBlock;
  int qsub = 0;
  if (mq > 1) {
    qsub = x % mq;
    x /= mq;
  }
  if (a.xcd_round > 0) {
    const int R = a.xcd_round;
    const int r = x / R, u = x - r * R;
    x = r * R + (u & 7) * (R >> 3) + (u >> 3);
  }
  // the item's head index counts packs of HPW consecutive heads of one KV
  // group (wph < 4: 4 / wph heads per workgroup)
  const int wph = a.wph;
  const int HPW = WAVES / wph;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // a KV group's heads in packs of HPW; when G is not a multiple of HPW the
  // group's last pack is partial, and its spare waves take the group's last
  // head, load and synchronise like the others, and store nothing
  const int gpk = (a.G + HPW - 1) / HPW;  // packs per KV group
  const Item it = decode_item(x, a.bm, a.B, (a.Hq / a.G) * gpk);
  const PackedHead ph = packed_head(it.h, a.G, HPW, wave / wph);
  const int b = it.b, h = ph.h, hk = ph.hk;
  const bool hvalid = ph.valid;
  const int q_tile0 = it.qb * a.bm.QBS + qsub * kBlock;
  if (q_tile0 >= a.Q_LEN) return;  // a 128-row tile past Q_LEN (BLOCK_SIZE > 128)
  Lane<D> ln;
  ln.lane = threadIdx.x & 63;
  ln.l32 = ln.lane & 31;
  ln.hh = ln.lane >> 5;
  ln.vg = (ln.lane >> 4) & 1;
  ln.vi = ln.lane & 15;
  ln.c16 = ln.lane & 15;
  ln.g4 = ln.lane >> 4;
  ln.q = R16 ? q_tile0 + ln.c16 : q_tile0 + (wave % wph) * 32 + ln.l32;
  const bool qvalid = hvalid && ln.q < a.Q_LEN;  // also gates every store
  ln.qc = qvalid ? ln.q : a.Q_LEN - 1;
  // document ids (COMPOSITE: only when a term tests documents)
  const int* doc_row =
      (mask_uses_doc(MASK) && a.mp.doc) ? a.mp.doc + b * a.mp.doc_bstride : nullptr;
  ln.dq = doc_row ? doc_row[ln.qc] : 0;
  ln.qw_lo = __builtin_amdgcn_readfirstlane(ln.qc);
  ln.qw_hi = __builtin_amdgcn_readlane(ln.qc, 31);
  if constexpr (R16) ln.init_offsets16();
  else ln.init_offsets();
  ln.slope2 = 0.0f;
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
    ln.slope2 = alibi_slope(a.slopes, h, a.Hq) * kLog2e;

  BlockLoader<D, false, WAVES> kload;
  BlockLoader<D, true, WAVES> vload;
  constexpr bool paged = PAGED;
  kload.init(a.k + (paged ? 0 : b * a.sk0) + hk * a.sk1, a.sk2, wave, ln.lane, sK0);
  vload.init(a.v + (paged ? 0 : b * a.sv0) + hk * a.sv1, a.sv2, wave, ln.lane, sV0);
  // paged KV: physical page of the logical key kv0 (clamped into the cache,
  // so a bad page table computes garbage but never reads outside it), and
  // loader bases that put logical key kv0's row of that page at
  // base + kv0 * row_bytes, so the per-step address arithmetic is unchanged
  const unsigned long long kbase0 = kload.base, vbase0 = vload.base;
  auto phys_page = [&](int kv0) {
    // a key tile past KV_LEN (loads nothing) reads the last page's entry
    const int lp = min(kv0, a.KV_LEN - 1) / a.page_size;
    const int pp = a.page_table[(long long)b * a.pt_stride + lp];
    return min(max(pp, 0), a.num_pages - 1);
  };
  auto set_page = [&](int kv0, int pp) {
    const long long first = (long long)(kv0 / a.page_size) * a.page_size;
    kload.base = kbase0 + (unsigned long long)(2 * pp * a.sk0 - first * kload.row_bytes);
    vload.base = vbase0 + (unsigned long long)(2 * pp * a.sv0 - first * vload.row_bytes);
  };
  const unsigned k_lds[2] = {kload.lds0, kload.lds0 + (lds_addr(sK1) - lds_addr(sK0))};
  const unsigned v_lds[2] = {vload.lds0, vload.lds0 + (lds_addr(sV1) - lds_addr(sV0))};

  const long long lrow = (long long)it.mrow * a.bm.NKB;
  // counts are clamped to the list length so a malformed BlockMask cannot
  // index past the staged list; the first entry of each list is read with
  // the counts, so the first step's loads need not wait for the staging
  const int nfull_c = __builtin_amdgcn_readfirstlane(min(a.bm.full_num[it.mrow], a.bm.NKB));
  const int n_c = __builtin_amdgcn_readfirstlane(min(nfull_c + a.bm.kv_num[it.mrow], a.bm.NKB));
  // in 128-key tiles: listed tile i covers 128-key tiles [i * mk, i * mk + mk)
  const int nfull = nfull_c * mk, n = n_c * mk;
  const int nlist = a.bm.NKB * mk;  // 128-key tiles the lists can name
  // this workgroup's slice [t_begin, t_end) of the item's tiles
  const int t_begin = (int)((long long)n * split / a.splits);
  const int t_end = (int)((long long)n * (split + 1) / a.splits);
  // Walk order (position t -> 128-key tile index). ALiBi scores grow toward
  // the diagonal, so an ascending walk raised the reference max (a rescale
  // of O) on almost every step of a steep head; the ALiBi kinds walk the
  // partial tiles, then the full ones, each by descending key, so causal rows
  // start on their diagonal tile and the maximum is known from the first
  // step. The other kinds walk the full tiles, then the partial ones, by
  // ascending key; masks whose lowest partial tile can leave a whole 64-key
  // step unattended (a sliding window's sink tile, a PrefixLM prefix tile)
  // walk their partial tiles by descending key instead, so that tile comes
  // last and its second step can be cut (see the half tile below).
  constexpr bool kDesc = SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI;
  constexpr bool kHalfLast = SPT == 2 && !kDesc &&
      (MASK == MASK_SLIDING_SINK || MASK == MASK_PREFIX_LM || MASK == MASK_COMPOSITE);
  const int npart = n - nfull;
  auto listed = [&](int t) {
    if constexpr (kDesc) {
      const bool part = t < npart;
      const int u = part ? npart - 1 - t : n - 1 - t;  // ascending piece of its list
      const int c = u / mk;
      const int idx =
          part ? a.bm.kv_idx[lrow + min(c, a.bm.NKB - 1)] : a.bm.full_idx[lrow + c];
      return idx * mk + (u - c * mk);
    } else if constexpr (kHalfLast) {
      const bool part = t >= nfull;
      const int u = part ? n - 1 - t : t;  // ascending piece of its list
      const int c = u / mk;
      const int idx =
          part ? a.bm.kv_idx[lrow + min(c, a.bm.NKB - 1)] : a.bm.full_idx[lrow + c];
      return idx * mk + (u - c * mk);
    } else {
      const int c = t / mk;
      const int idx = c < nfull_c ? a.bm.full_idx[lrow + c]
                                  : a.bm.kv_idx[lrow + min(c - nfull_c, a.bm.NKB - 1)];
      return idx * mk + (t - c * mk);
    }
  };
  const int first_tile = listed(t_begin);
  // the item's tiles in walk order, staged in LDS once (paged KV: and each
  // tile's physical page, after the tile list)
  int* tpage = tlist + ((nlist + 3) & ~3);
  for (int t = threadIdx.x; t < n; t += THREADS) {
    const int idx = listed(t);
    tlist[t] = idx;
    if constexpr (paged) tpage[t] = phys_page(kBlock * min(max(idx, 0), nlist - 1));
  }
  // document ids of a step's keys -> docbuf (rows past KV_LEN read as 0)
  auto issue_doc = [&](int buf, int kv0) {
    if constexpr (mask_uses_doc(MASK)) {
      if (wave == 0 && doc_row) {
        const int rows = min(a.KV_LEN, a.doc_len) - kv0;
        const i32x4 rsrc = make_rsrc(reinterpret_cast<unsigned long long>(doc_row + kv0),
                                     rows > 0 ? 4u * (unsigned)rows : 0u);
#pragma unroll
        for (int c = 0; c < DOC_STRIDE / 64; ++c)
          dma4(rsrc, __builtin_amdgcn_readfirstlane(lds_addr(docbuf + buf * DOC_STRIDE + 64 * c)),
               4 * ln.lane + 256 * c);
      }
    }
  };

  f32x16 o[R16 ? 1 : G::DB];  // O^T accumulators, 32-row layout
  f32x4 o16[R16 ? D / 16 : 1];  // 16-row layout
#pragma unroll
  for (int i = 0; i < (R16 ? 1 : G::DB); ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
#pragma unroll
  for (int i = 0; i < (R16 ? D / 16 : 1); ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) o16[i][r] = 0.0f;
  float m_ref = -INFINITY;
  float l = 0.0f;   // row sum of the probabilities (fp32): the LSE
  float lp = 0.0f;  // row sum of the rounded probabilities P.V multiplies: O's divisor

  if (t_end > t_begin) {
    // tile indices are clamped into [0, NKB): a malformed BlockMask computes
    // garbage but never reads outside the KV tensors
    auto clamp_kv0 = [&](int idx) { return kBlock * min(max(idx, 0), nlist - 1); };
    auto tile_kv0 = [&](int t) { return clamp_kv0(__builtin_amdgcn_readfirstlane(tlist[t])); };
    // prologue: step 0 -> buffer 0, Q^T fragments; then the tile list is
    // visible (barrier in wait_loads_and_sync)
    int kv0 = clamp_kv0(__builtin_amdgcn_readfirstlane(first_tile));
    if constexpr (paged) set_page(kv0, __builtin_amdgcn_readfirstlane(phys_page(kv0)));
    issue_doc(0, kv0);
    kload.issue(kv0, a.KV_LEN, k_lds[0]);
    vload.issue(kv0, a.KV_LEN, v_lds[0]);
    typename E::V8 qf[G::KS];
    {
      const u16* qrow = a.q + b * a.sq0 + h * a.sq1 + (long long)ln.qc * a.sq2;
      if constexpr (R16) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
          qf[ks] = as_v8<F16>(*reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * ln.g4));
      } else {
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks)
          qf[ks] = as_v8<F16>(*reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * ln.hh));
      }
    }
    wait_loads_and_sync();

    // Step g (global step counter over all tiles) reads buffer g % 2; at its
    // start it issues the loads of step g + 1 into the other buffer (read by
    // step g - 1, which every wave finished before the last barrier).
    int g = 0;
    int t_next = t_begin + 1;
    int kv_tile_next = t_next < t_end ? tile_kv0(t_next) : 0;
    auto tile_page = [&](int t) {
      return (paged && t < t_end) ? __builtin_amdgcn_readfirstlane(tpage[t]) : 0;
    };
    int pg_next = tile_page(t_next);
    // The walk's last tile, when partial, may have a second step that no
    // row of the workgroup attends (a sliding window's sink tile for rows
    // past the window): a workgroup-wide vote before the walk.
    bool half_last = false;
    if constexpr (kHalfLast) {
      const int tl = t_end - 1;
      const int kv_half = tile_kv0(tl) + NK;
      const bool may = step_may_attend<MASK>(
          mask_limits<D, MASK>(kv_half + 4 * (R16 ? ln.g4 : ln.hh), a, ln), NK);
      half_last = (tl >= nfull) && !__syncthreads_or(may);
    }
    auto run_tile = [&](auto masked_tag) {
#pragma unroll
      for (int sub = 0; sub < SPT; ++sub) {
        constexpr bool M = decltype(masked_tag)::value;
        // the item's last tile when its second step is masked for every row
        // of the workgroup (say a sliding window's sink tile): skip that
        // step; nothing follows it, so the buffer parity does not matter
        if constexpr (M && kHalfLast)
          if (sub == 1 && half_last && t_next == t_end) break;
        const bool last_sub = sub == SPT - 1;
        const bool has_next = !last_sub || t_next < t_end;
        const int kv_nxt = last_sub ? kv_tile_next : kv0 + NK;
        // buffer of this step: with two steps per tile the parity is the
        // sub-step (every tile starts on buffer 0)
        const int cur = (SPT == 2) ? sub : (g & 1);
        const int nb = cur ^ 1;
        if (has_next) issue_doc(nb, kv_nxt);
        if constexpr (paged)
          if (last_sub && has_next) set_page(kv_nxt, pg_next);
        // without a next step the loads get an empty range (they fetch
        // nothing; buffer nb was last read before the previous barrier)
        constexpr int KPW = decltype(kload)::KB_PER_WAVE;
        const i32x4 krs = kload.plan(has_next ? kv_nxt : a.KV_LEN, a.KV_LEN);
        const i32x4 vrs = vload.plan(has_next ? kv_nxt : a.KV_LEN, a.KV_LEN);
        auto dma = [&](int i) {
          if (i < KPW) kload.issue_one(krs, k_lds[nb], i);
          else vload.issue_one(vrs, v_lds[nb], i - KPW);
        };
        if constexpr (R16)
          step16<D, MASK, SCORE, M, 2 * KPW, F16>(
              o16, m_ref, l, lp, qf, cur ? sK1 : sK0, cur ? sV1 : sV0, kv0,
              mask_uses_doc(MASK) ? docbuf + cur * DOC_STRIDE : nullptr, a, ln, dma);
        else
          step<D, MASK, SCORE, M, 2 * KPW, F16>(
              o, m_ref, l, lp, qf, cur ? sK1 : sK0, cur ? sV1 : sV0, kv0,
              mask_uses_doc(MASK) ? docbuf + cur * DOC_STRIDE : nullptr, a, ln, dma);
        kv0 = kv_nxt;
        ++g;
        wait_loads_and_sync();
      }
      ++t_next;
      kv_tile_next = t_next < t_end ? tile_kv0(t_next) : 0;
      pg_next = tile_page(t_next);
    };
    // partial tiles take the masked path, full tiles the unmasked one; a
    // full tile crossing KV_LEN (never listed by the builder; the highest
    // full tile) is masked on the key bound
    int j = t_begin;
    if constexpr (kDesc) {
      const int mask_end =
          (nfull > 0 && tile_kv0(npart) + kBlock > a.KV_LEN) ? npart + 1 : npart;
      for (; j < min(mask_end, t_end); ++j) run_tile(std::true_type{});
      for (; j < t_end; ++j) run_tile(std::false_type{});
    } else {
      const int nfull_fast =
          (nfull > 0 && tile_kv0(nfull - 1) + kBlock > a.KV_LEN) ? nfull - 1 : nfull;
      for (; j < min(nfull_fast, t_end); ++j) run_tile(std::false_type{});
      for (; j < t_end; ++j) run_tile(std::true_type{});
    }
  }

  if constexpr (R16) {
    // 16-row epilogue: a query's row sum is spread over four lanes; lane
    // holds O^T rows 16*db + 4*g4 + r of query c16
    const float l1 = l + __shfl_xor(l, 16, 64);
    const float l_tot16 = l1 + __shfl_xor(l1, 32, 64);
    const float lp0 = kRoundedSum<SCORE> ? lp : l;
    const float lp1 = lp0 + __shfl_xor(lp0, 16, 64);
    const float lp_tot16 = lp1 + __shfl_xor(lp1, 32, 64);
    const float inv16 = lp_tot16 > 0.0f ? 1.0f / lp_tot16 : 0.0f;
    const float lse2 = l_tot16 > 0.0f ? (m_ref + fast_log2(l_tot16)) * kLn2 : -INFINITY;
    if (!qvalid) return;
    auto put_f32 = [&](float* orow) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        float4 v4;
        v4.x = o16[db][0] * inv16;
        v4.y = o16[db][1] * inv16;
        v4.z = o16[db][2] * inv16;
        v4.w = o16[db][3] * inv16;
        *reinterpret_cast<float4*>(orow + 16 * db + 4 * ln.g4) = v4;
      }
    };
    if (a.splits > 1) {
      const long long row = (((long long)split * a.B + b) * a.Hq + h) * a.Q_LEN + ln.q;
      put_f32(a.part_o + row * D);
      if (ln.g4 == 0) a.part_lse[row] = lse2;
      return;
    }
    if (a.o32) put_f32(a.o32 + (((long long)b * a.Hq + h) * a.Q_LEN + ln.q) * D);
    u16* orow = a.o + b * a.so0 + h * a.so1 + (long long)ln.q * a.so2;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      typename E::V4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) pk[j] = (typename E::T)(o16[db][j] * inv16);
      *reinterpret_cast<typename E::V4*>(orow + 16 * db + 4 * ln.g4) = pk;
    }
    if (ln.g4 == 0) a.lse[((long long)b * a.Hq + h) * a.Q_LEN + ln.q] = lse2;
    return;
  }

  // epilogue: O = O_acc / l, LSE = ln(sum) + max
  // O is divided by the sum of the rounded probabilities it was accumulated
  // from for the score-mod kinds (see kRoundedSum), else by the fp32 sum;
  // LSE takes the fp32 sum
  const float l_tot = l + __shfl_xor(l, 32, 64);
  const float lp_tot = kRoundedSum<SCORE> ? lp + __shfl_xor(lp, 32, 64) : l_tot;
  const float inv = lp_tot > 0.0f ? 1.0f / lp_tot : 0.0f;
  if (a.splits > 1) {
    // this slice's normalised O and LSE (-inf for an empty slice), fp32
    if (qvalid) {
      const long long row = (((long long)split * a.B + b) * a.Hq + h) * a.Q_LEN + ln.q;
      float* orow = a.part_o + row * D;
#pragma unroll
      for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float4 v4;
          v4.x = o[db][4 * gq + 0] * inv;
          v4.y = o[db][4 * gq + 1] * inv;
          v4.z = o[db][4 * gq + 2] * inv;
          v4.w = o[db][4 * gq + 3] * inv;
          *reinterpret_cast<float4*>(orow + 32 * db + 8 * gq + 4 * ln.hh) = v4;
        }
      if (ln.hh == 0)
        a.part_lse[row] = l_tot > 0.0f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  if (qvalid && a.o32) {
    float* orow = a.o32 + (((long long)b * a.Hq + h) * a.Q_LEN + ln.q) * D;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float4 v4;
        v4.x = o[db][4 * gq + 0] * inv;
        v4.y = o[db][4 * gq + 1] * inv;
        v4.z = o[db][4 * gq + 2] * inv;
        v4.w = o[db][4 * gq + 3] * inv;
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * gq + 4 * ln.hh) = v4;
      }
  }
  if (qvalid) {
    u16* orow = a.o + b * a.so0 + h * a.so1 + (long long)ln.q * a.so2;
#pragma unroll
    for (int db = 0; db < G::DB; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        typename E::V4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = (typename E::T)(o[db][4 * gq + j] * inv);
        *reinterpret_cast<typename E::V4*>(orow + 32 * db + 8 * gq + 4 * ln.hh) = pk;
      }
    }
    if (ln.hh == 0) {
      const float lse = l_tot > 0.0f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
      a.lse[((long long)b * a.Hq + h) * a.Q_LEN + ln.q] = lse;
    }
  }
}

template <int D, int MASK, int SCORE, bool PAGED, bool F16, bool R16>
hipError_t launch_one(const FwdArgs& args, int grid, hipStream_t stream) {
  const int nlist = args.bm.NKB * (args.bm.BS / kBlock);
  const int lds = 4 * ((nlist + 3) & ~3) * (PAGED ? 2 : 1);
  const void* fn = reinterpret_cast<const void*>(&fwd_bf16_kernel<D, MASK, SCORE, PAGED, F16, R16>);
  // The kernel's dynamic-LDS limit is raised once per device to everything
  // the CU has beside its static LDS; the value is the same for every call,
  // so concurrent first calls at worst set it twice, never lower it.
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> raised[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= kMaxDevices || !raised[dev].load(std::memory_order_acquire)) {
    hipFuncAttributes attr;
    e = hipFuncGetAttributes(&attr, fn);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxLdsBytes - (int)attr.sharedSizeBytes);
    if (e != hipSuccess) return e;
    if (dev < kMaxDevices) raised[dev].store(true, std::memory_order_release);
  }
  fwd_bf16_kernel<D, MASK, SCORE, PAGED, F16, R16><<<grid, 64 * kWavesPerHead, lds, stream>>>(args);
  return hipGetLastError();
}

template <int D, int MASK, bool PAGED, bool F16, bool R16>
hipError_t dispatch_score(const FwdArgs& args, int score, int grid, hipStream_t stream) {
  switch (score) {
    case SCORE_NONE:
      return launch_one<D, MASK, SCORE_NONE, PAGED, F16, R16>(args, grid, stream);
    case SCORE_ALIBI:
      return launch_one<D, MASK, SCORE_ALIBI, PAGED, F16, R16>(args, grid, stream);
    case SCORE_SOFTCAP:
      return launch_one<D, MASK, SCORE_SOFTCAP, PAGED, F16, R16>(args, grid, stream);
    case SCORE_SOFTCAP_ALIBI:
      return launch_one<D, MASK, SCORE_SOFTCAP_ALIBI, PAGED, F16, R16>(args, grid, stream);
    default:
      return launch_one<D, MASK, SCORE_SCALED, PAGED, F16, R16>(args, grid, stream);
  }
}

template <int D, bool PAGED, bool F16, bool R16>
hipError_t dispatch_mask(const FwdArgs& args, int mask, int score, int grid, hipStream_t stream) {
  switch (mask) {
    case MASK_NOOP:
      return dispatch_score<D, MASK_NOOP, PAGED, F16, R16>(args, score, grid, stream);
    case MASK_CAUSAL:
      return dispatch_score<D, MASK_CAUSAL, PAGED, F16, R16>(args, score, grid, stream);
    case MASK_SLIDING_SINK:
      return dispatch_score<D, MASK_SLIDING_SINK, PAGED, F16, R16>(args, score, grid, stream);
    case MASK_PREFIX_LM:
      return dispatch_score<D, MASK_PREFIX_LM, PAGED, F16, R16>(args, score, grid, stream);
    case MASK_COMPOSITE:
      return dispatch_score<D, MASK_COMPOSITE, PAGED, F16, R16>(args, score, grid, stream);
    default:
      return dispatch_score<D, MASK_DOCUMENT, PAGED, F16, R16>(args, score, grid, stream);
  }
}

template <int D, bool PAGED, bool F16>
hipError_t dispatch_step(const FwdArgs& args, bool r16, int mask, int score, int grid,
                         hipStream_t stream) {
  if constexpr (D <= 128)
    if (r16) return dispatch_mask<D, PAGED, F16, true>(args, mask, score, grid, stream);
  return dispatch_mask<D, PAGED, F16, false>(args, mask, score, grid, stream);
}

// One (head dim, KV layout, element type) slice of the kernel instantiations:
// every mask kind x score kind x MFMA step. fwd_bf16_inst.hip holds the
// explicit instantiations (one object file per slice, compiled in
// parallel); the launcher only declares them.
template <int D, bool PAGED, bool F16>
hipError_t fwd16_launch(const FwdArgs& a, bool r16, int mask, int score, int grid,
                        hipStream_t stream) {
  return dispatch_step<D, PAGED, F16>(a, r16, mask, score, grid, stream);
}

#define FA_FWD16_SLICE(D, PAGED, F16)                                                        \
  template hipError_t fwd16_launch<D, PAGED, F16>(const FwdArgs&, bool, int, int, int,     \
                                                  hipStream_t)
#define FA_FWD16_SLICES(prefix)                                                              \
  prefix FA_FWD16_SLICE(64, false, false); prefix FA_FWD16_SLICE(128, false, false);        \
  prefix FA_FWD16_SLICE(256, false, false); prefix FA_FWD16_SLICE(64, true, false);         \
  prefix FA_FWD16_SLICE(128, true, false); prefix FA_FWD16_SLICE(256, true, false);         \
  prefix FA_FWD16_SLICE(64, false, true); prefix FA_FWD16_SLICE(128, false, true);          \
  prefix FA_FWD16_SLICE(256, false, true); prefix FA_FWD16_SLICE(64, true, true);           \
  prefix FA_FWD16_SLICE(128, true, true); prefix FA_FWD16_SLICE(256, true, true)

}  // namespace fa
