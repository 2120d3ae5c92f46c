// Shared device-side definitions for the gfx950 block-sparse attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kBlock = 128;  // BlockMask tile edge (queries and keys)

// Kinds, mirrored from the C header's enums (kept numeric so kernels can be
// templated on them).
enum MaskKind : int {
  MASK_NOOP = 0,
  MASK_CAUSAL = 1,
  MASK_SLIDING_SINK = 2,
  MASK_DOCUMENT = 3,
  MASK_PREFIX_LM = 4,
  MASK_COMPOSITE = 5  // OR of up to 4 terms, each an AND of primitives
};

// Primitives of a composite mask term (bit set = the term requires it).
enum MaskPrim : int {
  PRIM_CAUSAL = 1,    // kv <= q
  PRIM_WINDOW = 2,    // q - kv < window
  PRIM_SINK = 4,      // kv < sinks
  PRIM_PREFIX = 8,    // kv < prefix
  PRIM_DOCUMENT = 16  // doc[q] == doc[kv]
};
constexpr int kMaxTerms = 4;

// Kinds whose kernels read document ids.
constexpr bool mask_uses_doc(int kind) { return kind == MASK_DOCUMENT || kind == MASK_COMPOSITE; }
enum ScoreKind : int { SCORE_NONE = 0, SCORE_ALIBI = 1, SCORE_SOFTCAP = 2, SCORE_SOFTCAP_ALIBI = 3 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Mask parameters as the kernels see them. `doc` already points at batch
// row 0; `doc_bstride` is 0 when one document row is shared by all batches.
struct MaskParams {
  int window;
  int sinks;
  const int* doc;
  long long doc_bstride;
  int prefix;  // PREFIX_LM: keys [0, prefix) are visible to every query
  // COMPOSITE: allowed = OR over terms[0 .. nterms) of (AND of the term's
  // primitives); a term with no bits allows everything
  int nterms;
  int terms[kMaxTerms];
};

// Keys [lo, hi] a composite term's interval primitives allow for query q
// (the document primitive is tested separately; lo > hi when none).
__device__ __forceinline__ void term_interval(int bits, int q, const MaskParams& p, int& lo,
                                              int& hi) {
  lo = 0;
  hi = 0x7fffffff;
  if (bits & PRIM_CAUSAL) hi = min(hi, q);
  if (bits & PRIM_WINDOW) lo = max(lo, q - p.window + 1);
  if (bits & PRIM_SINK) hi = min(hi, p.sinks - 1);
  if (bits & PRIM_PREFIX) hi = min(hi, p.prefix - 1);
}

// Composite mask of one element; dq / dkv are the document ids of the query
// and key (read only when a term has the document primitive).
// Evaluated without branches: every term slot is tested and the unused ones
// are masked out, so a per-element test compiles to compares and selects.
__device__ __forceinline__ bool composite_allowed(const MaskParams& p, int q, int kv, int dq,
                                                  int dkv) {
  bool any = false;
#pragma unroll
  for (int t = 0; t < kMaxTerms; ++t) {
    const int bits = p.terms[t];
    int lo, hi;
    term_interval(bits, q, p, lo, hi);
    const bool in = (kv >= lo) & (kv <= hi) & ((bits & PRIM_DOCUMENT) == 0 | dq == dkv);
    any = any | (in & (t < p.nterms));
  }
  return any;
}

// The BlockMask as the forward reads it.
struct BlockMaskView {
  const int* kv_num;    // [Bm][Hm][NQB]
  const int* kv_idx;    // [Bm][Hm][NQB][NKB]
  const int* full_num;  // [Bm][Hm][NQB]
  const int* full_idx;  // [Bm][Hm][NQB][NKB]
  const int* schedule;  // [Bm*Hm*NQB]
  int Bm, Hm, NQB, NKB;
  int BS = kBlock;   // KV_BLOCK_SIZE of the lists (a multiple of kBlock)
  int QBS = kBlock;  // Q_BLOCK_SIZE of the lists (a multiple of kBlock)
};

// Element mask of each kind: allowed(b, q, kv) for in-range indices.
template <int KIND>
struct Mask;

template <>
struct Mask<MASK_NOOP> {
  __device__ __forceinline__ static bool allowed(const MaskParams&, const int*, int, int) {
    return true;
  }
};

template <>
struct Mask<MASK_CAUSAL> {
  __device__ __forceinline__ static bool allowed(const MaskParams&, const int*, int q, int kv) {
    return kv <= q;
  }
};

template <>
struct Mask<MASK_SLIDING_SINK> {
  __device__ __forceinline__ static bool allowed(const MaskParams& p, const int*, int q, int kv) {
    return kv <= q && ((q - kv) < p.window || kv < p.sinks);
  }
};

template <>
struct Mask<MASK_PREFIX_LM> {
  __device__ __forceinline__ static bool allowed(const MaskParams& p, const int*, int q, int kv) {
    return kv <= q || kv < p.prefix;
  }
};

template <>
struct Mask<MASK_COMPOSITE> {
  // doc: this batch's document id row (nullptr when no term uses it)
  __device__ __forceinline__ static bool allowed(const MaskParams& p, const int* doc, int q,
                                                 int kv) {
    return composite_allowed(p, q, kv, doc ? doc[q] : 0, doc ? doc[kv] : 0);
  }
};

template <>
struct Mask<MASK_DOCUMENT> {
  // doc: this batch's document id row.
  __device__ __forceinline__ static bool allowed(const MaskParams&, const int* doc, int q, int kv) {
    return (kv <= q) & (doc[q] == doc[kv]);  // both ids in range: no short circuit needed
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Score modification in the base-2 domain. `s` is the raw dot product q.k;
// the result is log2(e) * score_mod(scale * s), so exp2 of it is exp of the
// modified score.
//   c_scale  = scale * log2(e)
//   c_cap    = 2 * scale * log2(e) / softcap       (tanh argument, doubled)
//   cap2     = softcap * log2(e)
//   slope2   = m_h * log2(e)
template <int SCORE>
struct ScoreMod {
  __device__ __forceinline__ static float apply(float s, float c_scale, float c_cap, float cap2,
                                                float slope2, float dist) {
    float x;
    if constexpr (SCORE == SCORE_SOFTCAP || SCORE == SCORE_SOFTCAP_ALIBI) {
      // softcap * tanh(y) with tanh(y) = 1 - 2 / (exp(2y) + 1)
      float e = fast_exp2(s * c_cap);
      float r = fast_rcp(e + 1.0f);
      x = fmaf(r, -2.0f * cap2, cap2);
    } else {
      x = s * c_scale;
    }
    if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI) {
      x = fmaf(slope2, dist, x);
    }
    return x;
  }
};

}  // namespace fa
