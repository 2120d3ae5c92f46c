// Block-sparse attention backward, bf16 or fp16 inputs, fp32 accumulation,
// gfx950. The build compiles this file once per element type (FA_BWD_F16 = 0
// for bf16, 1 for fp16), each object defining its launcher.
//
// Gradients of the forward in fwd_bf16.hip for an upstream dO, visiting only
// the tiles a BlockMask lists and applying mask_mod on partial tiles only
// (page "tensorplay.nn.attention API", section BlockMask, "Details": items 1
// and 2 for the query-tile walk of dQ, items 3 and 4 for the KV-tile walk of
// dK and dV along the query dimension). With the scaled score s = scale * q.k,
// x = score_mod(s), P = exp(x - LSE) and Delta_i = sum_j P_ij dP_ij:
//
//   dV_j = sum_i P_ij dO_i                 dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - Delta_i) dx/ds   (dx/ds = 1 - tanh^2 for the cap)
//   dQ_i = scale sum_j dS_ij k_j           dK_j = scale sum_i dS_ij q_i
//
// Three launches run on the caller's stream:
//   dq_kernel<DELTA>  one workgroup per (b, h, query tile), in the forward's
//                 schedule order, walking the KV tiles of the forward lists:
//                 Delta_i = sum_j P_ij dP_ij from fp32 P and dP. Delta equals
//                 dO_i . O_i, but O is stored in 16 bits and the difference
//                 dP - Delta cancels: taken from that O, Delta's rounding
//                 reaches tens of percent of some rows' dQ, taken this way
//                 it stays at the fp32 level;
//   dq_kernel     the same walk again for dQ;
//   dkdv_kernel   one workgroup per (b, KV head, KV tile); walks the query
//                 tiles of the backward lists for every query head of the
//                 GQA group, so dK / dV are summed in registers with a fixed
//                 order (deterministic, no atomics).
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, or _f16): an operand fragment is 8
// elements per lane, lane l holding row/column l%32 and k = 8*(l/32) .. +7; a result is 16
// fp32 per lane, register r holding row 8*(r/4) + 4*(l/32) + r%4 and column
// l%32. The 32x32 score tiles are produced with the key (dQ) or the query
// (dK/dV) on the lane axis, so P and dS pack straight into the B operand of
// the next product, whose A operand is read transposed from LDS
// (ds_read_b64_tr_b16) in the matching row order.
//
// Tiles are staged in LDS as row-major blocks with 8 elements of padding per
// row (272-byte rows at D = 128), double-buffered and filled by direct
// global->LDS loads while the previous block computes. The padding spreads
// the 16-byte row reads over the banks; the transposed 8-byte reads take the
// block's rows in an order (sigma32 for the keys of dQ, pi16 for the queries
// of dK/dV) whose rows read together fall in disjoint banks.
#include <atomic>
#include <cmath>

#include "common.hpp"
#include "fwd_common.hpp"
#include "launch.hpp"

#if !defined(FA_BWD_F16)
#error "compile bwd_bf16.hip with -DFA_BWD_F16=<0|1>"
#endif

namespace fa {
namespace {

typedef unsigned short u16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// The 16-bit element (bf16 for F16 = false, else fp16): both take the same
// fragment layouts and a 32x32x16 MFMA with fp32 accumulation; P and dS are
// rounded to it for the second products, dQ / dK / dV are stored in it.
template <bool F16>
struct BElem {
  using T = __bf16;
  using V8 = bf16x8;
  using V4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct BElem<true> {
  using T = _Float16;
  using V8 = f16x8;
  using V4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kThreads = 256;  // four waves
// keys per dQ step (one LDS buffer): 64 at D = 128, a whole 128-key tile at
// D = 64, whose steps would otherwise be barrier-bound; two step buffers of
// K and V then take 68 or 72 KiB, so two workgroups share a CU
template <int D>
constexpr int dq_step_keys() { return D == 64 ? 128 : 64; }
constexpr int kPad = 8;        // elements of padding per LDS row

struct BwdArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  const u16* dout;
  const float* lse;  // [B][Hq][Q_LEN]
  float* delta;      // [B][Hq][Q_LEN]
  const float* o32;  // fp32 O [B][Hq][Q_LEN][D] or nullptr
  u16* dq;
  u16* dk;
  u16* dv;
  long long sq[3], sk[3], sv[3], sdo[3], sdq[3], sdk[3], sdv[3];
  int B, Hq, Hkv, G, Q_LEN, KV_LEN;
  MaskParams mp;
  float scale, c_scale, c_cap, cap2;
  const float* slopes;
  BlockMaskView bm;
  const int* q_num;   // [Bm][Hm][NKB]
  const int* q_idx;   // [Bm][Hm][NKB][NQB]
  const int* fq_num;
  const int* fq_idx;
};

template <bool F16>
__device__ __forceinline__ typename BElem<F16>::V8 ld_frag(const u16* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  typename BElem<F16>::V8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// Transposed operand fragment of a row-major LDS block [row][LDR]: lane row
// d = 32*db + lane%32, slot t <-> block row 16*ks + 8*(t/4) + 4*(lane/32) + t%4.
// Each 16-lane group of a ds_read_b64_tr_b16 supplies the 8-byte pieces (row
// j/4, columns 4*(j%4) .. +3) of a 4-row x 16-column block and lane j gets
// column j of it.
template <int LDR, bool F16>
__device__ __forceinline__ typename BElem<F16>::V8 tr_frag(const u16* blk, int lane, int ks,
                                                          int db) {
  const int hh = lane >> 5, vg = (lane >> 4) & 1, vi = lane & 15;
  const int row = 16 * ks + 4 * hh + (vi >> 2);
  const int col = 32 * db + 16 * vg + 4 * (vi & 3);
  typename BElem<F16>::V4 part[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(blk + (row + 8 * ht) * LDR + col));
    __builtin_memcpy(&part[ht], &raw, 8);
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// Rows [r0, r0 + 128) of a [len][D] 16-bit matrix (row stride `ld` elements)
// into a padded LDS block; rows at or past `len` are zero. Branch-free (the
// row is clamped and the value zeroed) so each thread's loads are issued
// back to back, NB at a time, before any of them is waited for.
template <int D, int NB>
__device__ __forceinline__ void stage_rows(u16* lds, const u16* g, long long ld, int r0, int len,
                                           int tid) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  constexpr int LDR = D + kPad;
  constexpr int PER = kBlock * CH / kThreads;  // chunks per thread
  constexpr int BATCH = PER < NB ? PER : NB;
  static_assert(PER % BATCH == 0, "whole batches");
#pragma unroll 1
  for (int b0 = 0; b0 < PER; b0 += BATCH) {
    uint4 val[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int c = tid + (b0 + i) * kThreads;
      const int r = c / CH, ch = c % CH;
      const int rr = min(r0 + r, len - 1);
      val[i] = *reinterpret_cast<const uint4*>(g + (long long)rr * ld + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int c = tid + (b0 + i) * kThreads;
      const int r = c / CH, ch = c % CH;
      const bool in = r0 + r < len;
      uint4 w = val[i];
      w.x = in ? w.x : 0u;
      w.y = in ? w.y : 0u;
      w.z = in ? w.z : 0u;
      w.w = in ? w.w : 0u;
      *reinterpret_cast<uint4*>(lds + r * LDR + ch * 8) = w;
    }
  }
}

template <int MASK>
__device__ __forceinline__ bool allowed_el(const MaskParams& mp, int q, int kv, int dq, int dkv) {
  if constexpr (MASK == MASK_NOOP) {
    return true;
  } else if constexpr (MASK == MASK_CAUSAL) {
    return kv <= q;
  } else if constexpr (MASK == MASK_SLIDING_SINK) {
    return kv <= q && ((q - kv) < mp.window || kv < mp.sinks);
  } else if constexpr (MASK == MASK_PREFIX_LM) {
    return kv <= q || kv < mp.prefix;
  } else if constexpr (MASK == MASK_COMPOSITE) {
    return composite_allowed(mp, q, kv, dq, dkv);
  } else {
    return (kv <= q) & (dq == dkv);
  }
}

// Logit in base 2 (x = log2(e) * score_mod(scale * s), -inf where masked or
// out of range) and dx/d(scale*s) of the element (q, kv), s = q.k.
template <int MASK, int SCORE, bool MASKED>
__device__ __forceinline__ void logit_and_slope(float s, int q, int kv, int dq, int dkv,
                                                float slope2, const BwdArgs& a, float& x,
                                                float& dmod) {
  if constexpr (SCORE == SCORE_SOFTCAP || SCORE == SCORE_SOFTCAP_ALIBI) {
    // cap * tanh(y) = cap * (1 - 2 r), r = 1 / (exp(2y) + 1); 1 - tanh^2 = 4 r (1 - r)
    const float e = fast_exp2(s * a.c_cap);
    const float r = fast_rcp(e + 1.0f);
    x = fmaf(r, -2.0f * a.cap2, a.cap2);
    dmod = 4.0f * r * (1.0f - r);
  } else {
    x = s * a.c_scale;
    dmod = 1.0f;
  }
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
    x = fmaf(slope2, (float)(kv - q), x);
  if constexpr (MASKED) {
    const bool ok = q < a.Q_LEN && kv < a.KV_LEN && allowed_el<MASK>(a.mp, q, kv, dq, dkv);
    x = ok ? x : -INFINITY;
  }
}

// lse in base 2; +inf for rows with no allowed key (P = 0 there)
__device__ __forceinline__ float lse_base2(float lse) {
  return lse == -INFINITY ? INFINITY : lse * kLog2e;
}

// Direct global->LDS loads for the backward's K/V and Q/dO tiles. A buffer
// resource covers [base, base + bytes); loads past it read as zero. Each
// wave-wide buffer_load_dwordx4 ... lds writes 1 KiB of LDS: lane l's 16
// bytes land at M0 + 16 l. M0 is an operand bound to M0; the asm keeps the
// CDNA wait states itself (one after a scalar write of M0, five after a
// vector instruction wrote a scalar operand of a vector memory instruction),
// since the compiler's hazard recognizer does not look inside inline asm.
__device__ __forceinline__ unsigned lds_u32(const void* p) {
  return (unsigned)(unsigned long long)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}
// Bytes a resource must cover for `rows` rows of `row_bytes` stride and D
// 16-bit elements: up to the last valid row's data, so a row stride below
// the row length (0 for rows broadcast along the sequence) still reads every
// valid row; rows past the last read as zero when the stride is the row
// length or more, else other valid rows (their scores are masked either way).
__device__ __forceinline__ unsigned range_bytes(int rows, long long row_bytes, int D) {
  return rows > 0 ? (unsigned)((rows - 1) * row_bytes + 2 * D) : 0u;
}
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, unsigned lds, int voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               : : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds)));
}
__device__ __forceinline__ void lds_dma4(i32x4 rsrc, unsigned lds, int voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
               : : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds)));
}

// Key order of the dQ walk inside a 32-key block: block row m = 16 a + 8 b +
// 4 c + i (a, b, c in {0, 1}, i < 4) is key sigma32(m) = 16 a + 4 i + 2 b + c.
// The S^T product's A operand takes key sigma32(lane % 32) in row lane % 32,
// so result register r of lane l (row 8 (r / 4) + 4 (l / 32) + r % 4) is key
// 16 (r / 8) + 4 (r % 4) + 2 ((r / 4) % 2) + l / 32, and the transposed K
// reads take the keys in that order. Each 32-lane half of a transposed read
// then touches four keys whose 272-byte (D = 128) rows are 4 rows apart: their
// 64-byte pieces fall in disjoint LDS banks, where consecutive rows overlap.
// The 16 keys of a row read stay distinct modulo 16, as before.
__device__ __forceinline__ constexpr int sigma32(int m) {
  return (m & 16) | ((m & 3) << 2) | (((m >> 3) & 1) << 1) | ((m >> 2) & 1);
}

// dQ operand K^T (32x32x16, read transposed from the key-major LDS block):
// lane row d = 32 db + lane % 32, slot t <-> block row sigma32(16 (ks % 2) + 8 (t / 4)
// + 4 (lane / 32) + t % 4) of the 32-key block ks / 2.
template <int LDR, bool F16>
__device__ __forceinline__ typename BElem<F16>::V8 tr_frag_keys(const u16* blk, int lane, int ks,
                                                               int db) {
  const int hh = lane >> 5, vg = (lane >> 4) & 1, vi = lane & 15;
  const int row = 16 * ks + 4 * (vi >> 2) + hh;  // + 2 ht
  const int col = 32 * db + 16 * vg + 4 * (vi & 3);
  typename BElem<F16>::V4 part[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(blk + (row + 2 * ht) * LDR + col));
    __builtin_memcpy(&part[ht], &raw, 8);
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, h, query tile); wave w owns query rows
// 32w .. 32w+31 of the tile. Per 32-key block: S^T = K.Q^T and dP^T = V.dO^T
// (key rows on the register axis, query on the lane axis), dS^T, then
// dQ^T += K^T . dS^T with K read transposed from LDS. With DELTA the walk
// only sums P dP per query row and writes Delta.
// ---------------------------------------------------------------------------
template <int D, int MASK, int SCORE, bool DELTA, bool F16>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(BwdArgs a) {
  using E = BElem<F16>;
  using T = typename E::T;
  constexpr int LDR = D + kPad;
  constexpr int KS = D / 16, DB = D / 32;
  // K and V in steps of 64 (D = 128) or 128 keys, double-buffered in dynamic
  // LDS ([buf][K | V][kStepKeys][LDR]) and filled by direct global->LDS loads
  // while the previous step computes; the steps' document ids likewise
  // ([buf][kStepKeys]).
  constexpr int kStepKeys = dq_step_keys<D>();
  constexpr int SPT = kBlock / kStepKeys;  // steps per tile
  extern __shared__ __attribute__((aligned(16))) u16 dq_lds[];
  __shared__ __attribute__((aligned(16))) int sdoc[2][kStepKeys];

  // BLOCK_SIZE = mk * 128: mk 128-row items per tile row, mk 128-key tiles
  // per listed tile
  const int mk = a.bm.BS / kBlock, mq = a.bm.QBS / kBlock;
  const Item it = decode_item(blockIdx.x / mq, a.bm, a.B, a.Hq);
  const int b = it.b, h = it.h, hk = h / a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q_tile0 = it.qb * a.bm.QBS + (blockIdx.x % mq) * kBlock;
  if (q_tile0 >= a.Q_LEN) return;  // a 128-row piece past Q_LEN
  const int q = q_tile0 + wave * 32 + l32;
  const bool qvalid = q < a.Q_LEN;
  const int qc = qvalid ? q : a.Q_LEN - 1;

  typename E::V8 qf[KS], dof[KS];
  {
    const u16* qrow = a.q + b * a.sq[0] + h * a.sq[1] + (long long)qc * a.sq[2];
    const u16* grow = a.dout + b * a.sdo[0] + h * a.sdo[1] + (long long)qc * a.sdo[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = ld_frag<F16>(qrow + 16 * ks + 8 * hh);
      dof[ks] = ld_frag<F16>(grow + 16 * ks + 8 * hh);
    }
  }
  const long long rowid = ((long long)b * a.Hq + h) * a.Q_LEN + qc;
  const float lse2 = qvalid ? lse_base2(a.lse[rowid]) : INFINITY;
  const float dlt = DELTA ? 0.0f : a.delta[rowid];
  float psum = 0.0f;  // DELTA: this lane's share of sum_j P dP
  float slope2 = 0.0f;
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
    slope2 = alibi_slope(a.slopes, h, a.Hq) * kLog2e;
  const int* doc_row =
      (mask_uses_doc(MASK) && a.mp.doc) ? a.mp.doc + b * a.mp.doc_bstride : nullptr;
  const int dq_id = doc_row ? doc_row[qc] : 0;

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  const int NKB = a.bm.NKB;
  const long long lrow = (long long)it.mrow * NKB;
  const int nfull = min(max(a.bm.full_num[it.mrow], 0), NKB);
  const int npart = min(max(a.bm.kv_num[it.mrow], 0), NKB);
  const u16* kbase = a.k + b * a.sk[0] + hk * a.sk[1];
  const u16* vbase = a.v + b * a.sv[0] + hk * a.sv[1];

  // one step from buffer `buf` (keys kv0 ..): S^T, dP^T, dS^T, then
  // dQ^T += K^T . dS^T, per 32-key block
  auto step = [&](int kv0, int buf, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const u16* sK = dq_lds + buf * 2 * kStepKeys * LDR;
    const u16* sV = sK + kStepKeys * LDR;
    // (two 32-key blocks unrolled at D = 128; the four of a D = 64 step in a
    // loop, which keeps the D = 64 kernels at their old register use)
    constexpr int kBlkUnroll = kStepKeys == 64 ? 2 : 1;
#pragma unroll kBlkUnroll
    for (int blk = 0; blk < kStepKeys / 32; ++blk) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const u16* krow = sK + (32 * blk + sigma32(l32)) * LDR + 8 * hh;
      const u16* vrow = sV + (32 * blk + sigma32(l32)) * LDR + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = E::mfma(ld_frag<F16>(krow + 16 * ks), qf[ks], s);
        dp = E::mfma(ld_frag<F16>(vrow + 16 * ks), dof[ks], dp);
      }
      typename E::V8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // key sigma32(8 (r / 4) + 4 hh + r % 4) of the block
        const int kl = 32 * blk + 16 * (r >> 3) + 4 * (r & 3) + 2 * ((r >> 2) & 1) + hh;
        float x, dm;
        logit_and_slope<MASK, SCORE, MASKED>(s[r], q, kv0 + kl, dq_id,
                                             mask_uses_doc(MASK) ? sdoc[buf][kl] : 0, slope2, a,
                                             x, dm);
        const float p = fast_exp2(x - lse2);
        if constexpr (DELTA) psum = fmaf(p, dp[r], psum);
        else dsf[r >> 3][r & 7] = (T)(p * (dp[r] - dlt) * dm);
      }
      if constexpr (!DELTA) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = E::mfma(tr_frag_keys<LDR, F16>(sK, lane, 2 * blk + k2, db), dsf[k2],
                              acc[db]);
      }
    }
  };

  // Loads of a step's keys [kv0, kv0 + kStepKeys) into buffer `buf`: the padded block is
  // SPR 16-byte slots per row (D / 8 of data and one of padding); wave-wide
  // load I fills slots [64 I, 64 I + 64), lane l slot 64 I + l from that
  // slot's row and chunk (a padding slot repeats the row's last chunk). Keys
  // at or past KV_LEN are outside the resources and read as zero.
  constexpr int SPR = 2 * LDR / 16;
  constexpr int NINS = kStepKeys * SPR / 64;
  static_assert(kStepKeys * SPR % 64 == 0, "whole wave-wide loads");
  constexpr int IPW = (NINS + kThreads / 64 - 1) / (kThreads / 64);
  auto dma_step = [&](int kv0, int buf) __attribute__((always_inline)) {
    const int rows = max(min(a.KV_LEN - kv0, kStepKeys), 0);
    const long long rk = 2 * a.sk[2], rv = 2 * a.sv[2];  // row bytes
    const i32x4 rsk = buf_rsrc(kbase + (long long)kv0 * a.sk[2], range_bytes(rows, rk, D));
    const i32x4 rsv = buf_rsrc(vbase + (long long)kv0 * a.sv[2], range_bytes(rows, rv, D));
    const unsigned lk = lds_u32(dq_lds + buf * 2 * kStepKeys * LDR);
    const unsigned lv = lk + 2 * kStepKeys * LDR;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int I = wave + (kThreads / 64) * i;
      if (I < NINS) {
        const int slot = 64 * I + lane;
        const int row = slot / SPR, ch = min(slot % SPR, SPR - 2);
        lds_dma16(rsk, lk + 1024 * I, row * (int)rk + 16 * ch);
        lds_dma16(rsv, lv + 1024 * I, row * (int)rv + 16 * ch);
      }
    }
    if constexpr (mask_uses_doc(MASK)) {
      if (doc_row && wave == 0) {
        const i32x4 rsd = buf_rsrc(doc_row + kv0, 4u * (unsigned)rows);
#pragma unroll
        for (int c = 0; c < kStepKeys / 64; ++c)
          lds_dma4(rsd, lds_u32(&sdoc[buf][64 * c]), 4 * lane + 256 * c);
      }
    }
  };

  // Tile t of the walk: 128-key piece t % mk of listed tile t / mk.
  const int ntile = (nfull + npart) * mk;
  auto tile_kv0 = [&](int t) __attribute__((always_inline)) {
    const int c = t / mk;
    const bool full = c < nfull;
    const int kb = min(max(full ? a.bm.full_idx[lrow + c] : a.bm.kv_idx[lrow + c - nfull], 0),
                       NKB - 1);
    return kb * a.bm.BS + (t - c * mk) * kBlock;
  };
  if (ntile > 0) {
    int kv0 = tile_kv0(0);
    dma_step(kv0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    // Step g reads buffer g % 2 (with two steps per tile every tile starts on
    // buffer 0); at its start it issues the next step's loads into the other
    // buffer (read by step g - 1, which every wave finished before the last
    // barrier).
    int g = 0;
    for (int t = 0; t < ntile; ++t) {
      const bool full = t / mk < nfull && kv0 + kBlock <= a.KV_LEN;
      const int kv_next = t + 1 < ntile ? tile_kv0(t + 1) : 0;
#pragma unroll
      for (int sub = 0; sub < SPT; ++sub) {
        const int cur = SPT == 2 ? sub : (g & 1);
        if (sub + 1 < SPT) dma_step(kv0 + kStepKeys * (sub + 1), cur ^ 1);
        else if (t + 1 < ntile) dma_step(kv_next, cur ^ 1);
        if (full) step(kv0 + kStepKeys * sub, cur, std::false_type{});
        else step(kv0 + kStepKeys * sub, cur, std::true_type{});
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        ++g;
      }
      kv0 = kv_next;
    }
  }

  if constexpr (DELTA) {
    // the two lanes holding a query row (lane, lane ^ 32) split its keys
    const float tot = psum + __shfl_xor(psum, 32, 64);
    if (qvalid && hh == 0) a.delta[rowid] = tot;
    return;
  }
  if (qvalid) {
    u16* out = a.dq + b * a.sdq[0] + h * a.sdq[1] + (long long)q * a.sdq[2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        typename E::V4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = (T)(acc[db][4 * gq + j] * a.scale);
        *reinterpret_cast<typename E::V4*>(out + 32 * db + 8 * gq + 4 * hh) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup of eight waves per (b, KV head, 128-key tile); wave w
// owns keys 16w .. 16w+15 and uses v_mfma_f32_16x16x32 products, so a wave
// holds half the accumulators of a 32-key wave and two waves share each SIMD
// (one runs its matrix products while the other computes P and dS). For
// every query head of the group and every query tile of the backward lists,
// per 32-query block: S = Q.K^T and dP = dO.V^T as two 16-query tiles each
// (query on the register axis, key on the lane axis), then dV^T += dO^T . P
// and dK^T += Q^T . dS over the block's 32 queries, with dO and Q read
// transposed from LDS.
// 16x16x32 layout: operand slot t of lane l holds k = 8*(l/16) + t of
// row / column l%16; result register r of lane l holds row 4*(l/16) + r,
// column l%16. In the P and dS operands slot t stands for query
// 16*(t/4) + 4*(l/16) + t%4 of the block (the two S tiles' registers in
// order), and the transposed reads take the dO and Q rows in that order.
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 8;

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(typename BElem<F16>::V8 a, typename BElem<F16>::V8 b,
                                        f32x4 c) {
  if constexpr (F16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Query order of the dK/dV walk inside a 16-query tile: tile row i (the S
// product's A-operand row, and result row 4*(lane/16) + r) is query
// pi16(i) of the tile: rows 0..7 the even queries, rows 8..15 the odd ones.
// The padded LDS rows are 272 bytes (D = 128; 144 at D = 64) apart, so the
// 16 rows of a row read still fall in distinct banks, and each pair of
// 16-lane groups of a transposed read (eight rows, 32 bytes each) takes
// eight queries of one parity, whose 32-byte pieces then fill the 256 bytes
// of LDS banks once instead of overlapping pairwise as consecutive rows do.
__device__ __forceinline__ constexpr int pi16(int i) { return ((i & 7) << 1) | (i >> 3); }
__device__ __forceinline__ constexpr int pi16_inv(int r) { return (r >> 1) | ((r & 1) << 3); }

// Transposed 16x16x32 operand of a row-major LDS block [row][LDR]: lane row
// d = 16*dt + lane%16, slot t <-> block row r0 + 16*(t/4) + pi16(4*(lane/16) + t%4),
// the query order of the P and dS operands.
// In each 16-lane group lane j supplies the 8-byte piece (row j/4, columns
// 4*(j%4) .. +3) of a 4-row x 16-column block and receives column j.
template <int LDR, bool F16>
__device__ __forceinline__ typename BElem<F16>::V8 tr_frag16(const u16* blk, int lane, int r0,
                                                            int dt) {
  const int g4 = lane >> 4, j = lane & 15;
  const int row = r0 + pi16(4 * g4 + (j >> 2));
  const int col = 16 * dt + 4 * (j & 3);
  typename BElem<F16>::V4 part[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(blk + (row + 16 * ht) * LDR + col));
    __builtin_memcpy(&part[ht], &raw, 8);
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int D, int MASK, int SCORE, bool F16>
__global__ __launch_bounds__(64 * kKvWaves, 1) void dkdv_kernel(BwdArgs a) {
  using E = BElem<F16>;
  using T = typename E::T;
  constexpr int LDR = D + kPad;
  constexpr int KS = D / 32;  // k-steps of the S and dP products
  constexpr int DT = D / 16;  // 16-row d tiles of dK^T and dV^T
  // The query tiles (Q and dO) are double-buffered in dynamic LDS and
  // filled by direct global->LDS loads while the previous tile computes, so
  // no registers are held for them.
  static_assert(D <= 128, "two query-tile buffers fit the CU's LDS up to D = 128");
  extern __shared__ __attribute__((aligned(16))) u16 dyn_lds[];  // [buf][Q | dO][kBlock][LDR]
  const u16* sQ = dyn_lds;
  const u16* sG = dyn_lds + kBlock * LDR;
  __shared__ __attribute__((aligned(16))) float slse[kBlock];
  __shared__ __attribute__((aligned(16))) float sdel[kBlock];
  __shared__ int sdoc[kBlock];

  const int NKB = a.bm.NKB, NQB = a.bm.NQB;
  // KV-tile-major order: every (b, KV head) of tile 0 first, then tile 1, ...
  // Under causal-like masks the early KV tiles have the longest query lists,
  // so the launch runs longest first (one workgroup per CU at this size).
  const int nbh = a.B * a.Hkv;
  const int mk = a.bm.BS / kBlock;   // 128-key items per tile column
  const int mq = a.bm.QBS / kBlock;  // 128-row pieces per listed query tile
  const int kb = blockIdx.x / nbh;  // in 128-key tiles
  const int kbc = kb / mk;          // the BlockMask's tile column
  const int bh = blockIdx.x - kb * nbh;
  if (kb * kBlock >= a.KV_LEN) return;  // a 128-key piece past KV_LEN
  const int hk = bh % a.Hkv, b = bh / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int kv = kb * kBlock + wave * 16 + c16;
  const bool kvalid = kv < a.KV_LEN;
  const int kvc = kvalid ? kv : a.KV_LEN - 1;

  typename E::V8 kf[KS], vf[KS];
  {
    const u16* krow = a.k + b * a.sk[0] + hk * a.sk[1] + (long long)kvc * a.sk[2];
    const u16* vrow = a.v + b * a.sv[0] + hk * a.sv[1] + (long long)kvc * a.sv[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = ld_frag<F16>(krow + 32 * ks + 8 * g4);
      vf[ks] = ld_frag<F16>(vrow + 32 * ks + 8 * g4);
    }
  }
  const int* doc_row =
      (mask_uses_doc(MASK) && a.mp.doc) ? a.mp.doc + b * a.mp.doc_bstride : nullptr;
  const int dkv_id = doc_row ? doc_row[kvc] : 0;

  f32x4 acck[DT], accv[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    acck[i] = f32x4{};
    accv[i] = f32x4{};
  }

  // The walk: for each query head of the group, its full then partial query
  // tiles of this KV tile; heads with empty lists are skipped.
  struct Pos {
    int gi, t, nfull, npart;
    long long mrow;
  };
  auto first_from = [&](int gi) __attribute__((always_inline)) {
    Pos p{gi, 0, 0, 0, 0};
    for (; p.gi < a.G; ++p.gi) {
      const int h = hk * a.G + p.gi;
      const int bmi = a.bm.Bm == 1 ? 0 : b;
      const int hm = a.bm.Hm == 1 ? 0 : h;
      p.mrow = ((long long)bmi * a.bm.Hm + hm) * NKB + kbc;
      p.nfull = min(max(a.fq_num[p.mrow], 0), NQB);
      p.npart = min(max(a.q_num[p.mrow], 0), NQB);
      if (p.nfull + p.npart > 0) break;
    }
    return p;
  };
  // p.t counts 128-row pieces: listed tile p.t / mq, piece p.t % mq
  auto next_pos = [&](Pos p) __attribute__((always_inline)) {
    if (p.t + 1 < (p.nfull + p.npart) * mq) {
      ++p.t;
      return p;
    }
    return first_from(p.gi + 1);
  };
  auto tile_q0 = [&](const Pos& p) __attribute__((always_inline)) {
    const int c = p.t / mq;
    const bool full = c < p.nfull;
    const int qb = full ? a.fq_idx[p.mrow * NQB + c] : a.q_idx[p.mrow * NQB + c - p.nfull];
    return min(max(qb, 0), NQB - 1) * a.bm.QBS + (p.t - c * mq) * kBlock;
  };

  // The next tile's LSE, Delta and document ids are loaded into registers
  // while the current tile computes, then written to LDS (its Q and dO rows
  // go straight to LDS, see dma_tile).
  float pl = 0.0f, pd = 0.0f;
  int pdoc = 0;
  auto fetch = [&](const Pos& p) __attribute__((always_inline)) {
    const int h = hk * a.G + p.gi;
    const int q0 = tile_q0(p);
    if (tid < kBlock) {
      const long long lrow = ((long long)b * a.Hq + h) * a.Q_LEN + min(q0 + tid, a.Q_LEN - 1);
      pl = a.lse[lrow];
      pd = a.delta[lrow];
      if constexpr (mask_uses_doc(MASK))
        if (doc_row) pdoc = doc_row[min(q0 + tid, a.Q_LEN - 1)];
    }
  };
  auto commit = [&](int q0) __attribute__((always_inline)) {
    if (tid < kBlock) {
      // query tid of the tile at its tile-row position (see pi16)
      const bool in = q0 + tid < a.Q_LEN;
      const int at = (tid & ~15) | pi16_inv(tid & 15);
      slse[at] = in ? lse_base2(pl) : INFINITY;
      sdel[at] = in ? pd : 0.0f;
      if constexpr (mask_uses_doc(MASK)) sdoc[at] = in ? pdoc : -2;
    }
  };

  // Per 32-query block the products run in batches of four: first the S and
  // dP products of each 16-query tile, two k-steps a batch, then the dV and
  // dK products, two d tiles a batch. The operand fragments of each batch
  // are read from LDS one or two batches ahead of its products (scheduling
  // barriers keep that order), so the products do not wait on an LDS round
  // trip one by one.
  auto tile = [&](int q0, float slope2, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    using V8 = typename E::V8;
    const int qlane = q0 + 8 * (g4 & 1) + (g4 >> 1);
    constexpr int NSB = KS;          // S / dP batches: 2 tiles x KS / 2 k-step pairs
    constexpr int NBT = NSB + DT / 2;  // all batches
    // batches read ahead: two, or one for the score-mod kinds, whose P and
    // dS arithmetic needs the registers
    constexpr int AHEAD = SCORE == SCORE_NONE ? 2 : 1;
    static_assert(KS % 2 == 0 && DT % 2 == 0, "pairs of k-steps and d tiles");
#pragma unroll 1
    for (int qs = 0; qs < kBlock / 32; ++qs) {
      f32x4 s[2], dp[2];
      V8 pf, dsf;
      V8 fb[AHEAD + 1][4];
      auto load_b = [&](int k, V8 (&f)[4]) __attribute__((always_inline)) {
        if (k < NSB) {
          const int hq = k / (KS / 2), ks0 = 2 * (k % (KS / 2));
          const u16* qrow = sQ + (32 * qs + 16 * hq + pi16(c16)) * LDR + 8 * g4 + 32 * ks0;
          const u16* grow = sG + (32 * qs + 16 * hq + pi16(c16)) * LDR + 8 * g4 + 32 * ks0;
          f[0] = ld_frag<F16>(qrow);
          f[1] = ld_frag<F16>(grow);
          f[2] = ld_frag<F16>(qrow + 32);
          f[3] = ld_frag<F16>(grow + 32);
        } else {
          const int j0 = 2 * (k - NSB);
          f[0] = tr_frag16<LDR, F16>(sG, lane, 32 * qs, j0);
          f[1] = tr_frag16<LDR, F16>(sQ, lane, 32 * qs, j0);
          f[2] = tr_frag16<LDR, F16>(sG, lane, 32 * qs, j0 + 1);
          f[3] = tr_frag16<LDR, F16>(sQ, lane, 32 * qs, j0 + 1);
        }
      };
      auto mfma_b = [&](int k, V8 (&f)[4]) __attribute__((always_inline)) {
        if (k < NSB) {
          const int hq = k / (KS / 2), ks0 = 2 * (k % (KS / 2));
          if (ks0 == 0) {
            s[hq] = f32x4{};
            dp[hq] = f32x4{};
          }
          s[hq] = mfma16<F16>(f[0], kf[ks0], s[hq]);
          dp[hq] = mfma16<F16>(f[1], vf[ks0], dp[hq]);
          s[hq] = mfma16<F16>(f[2], kf[ks0 + 1], s[hq]);
          dp[hq] = mfma16<F16>(f[3], vf[ks0 + 1], dp[hq]);
        } else {
          const int j0 = 2 * (k - NSB);
          accv[j0] = mfma16<F16>(f[0], pf, accv[j0]);
          acck[j0] = mfma16<F16>(f[1], dsf, acck[j0]);
          accv[j0 + 1] = mfma16<F16>(f[2], pf, accv[j0 + 1]);
          acck[j0 + 1] = mfma16<F16>(f[3], dsf, acck[j0 + 1]);
        }
      };
#pragma unroll
      for (int k = 0; k < AHEAD; ++k) load_b(k, fb[k]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NBT; ++k) {
        if (k == NSB) {
          // P and dS of the block (the S / dP products are done)
#pragma unroll
          for (int hq = 0; hq < 2; ++hq) {
            const int ql0 = 32 * qs + 16 * hq + 4 * g4;
            const float4 l4 = *reinterpret_cast<const float4*>(slse + ql0);
            const float4 d4 = *reinterpret_cast<const float4*>(sdel + ql0);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x, dm;
              // query pi16(4 g4 + r) = 8 (g4 & 1) + (g4 >> 1) + 2 r of the tile
              logit_and_slope<MASK, SCORE, MASKED>(s[hq][r], qlane + 32 * qs + 16 * hq + 2 * r, kv,
                                                   mask_uses_doc(MASK) ? sdoc[ql0 + r] : 0,
                                                   dkv_id, slope2, a, x, dm);
              const float p = fast_exp2(x - lv[r]);
              pf[4 * hq + r] = (T)p;
              dsf[4 * hq + r] = (T)(p * (dp[hq][r] - dl[r]) * dm);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_b(k, fb[k % (AHEAD + 1)]);
        if (k + AHEAD < NBT) load_b(k + AHEAD, fb[(k + AHEAD) % (AHEAD + 1)]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Direct loads of one query tile's Q and dO rows into LDS buffer `buf`
  // (D <= 128). The padded block is SPR 16-byte slots per row (D / 8 of data
  // and one of padding); wave-wide load I fills slots [64 I, 64 I + 64), lane
  // l slot 64 I + l, from that slot's row and chunk (a padding slot repeats
  // the row's last chunk). Rows at or past Q_LEN are outside the resource
  // and read as zero.
  constexpr int SPR = 2 * LDR / 16;
  constexpr int NINS = kBlock * SPR / 64;
  static_assert(kBlock * SPR % 64 == 0, "whole wave-wide loads");
  constexpr int IPW = (NINS + kKvWaves - 1) / kKvWaves;
  auto dma_tile = [&](const Pos& p, int buf) __attribute__((always_inline)) {
    {  // (scope of the tile's resources)
      const int h = hk * a.G + p.gi;
      const int q0 = tile_q0(p);
      const int rows = max(min(a.Q_LEN - q0, kBlock), 0);
      const long long rq = 2 * a.sq[2], rg = 2 * a.sdo[2];  // row bytes
      const i32x4 rsq = buf_rsrc(a.q + b * a.sq[0] + h * a.sq[1] + (long long)q0 * a.sq[2],
                                 range_bytes(rows, rq, D));
      const i32x4 rsg = buf_rsrc(a.dout + b * a.sdo[0] + h * a.sdo[1] + (long long)q0 * a.sdo[2],
                                 range_bytes(rows, rg, D));
      const unsigned lq = lds_u32(dyn_lds + buf * 2 * kBlock * LDR);
      const unsigned lg = lq + 2 * kBlock * LDR;
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int I = wave + kKvWaves * i;
        if (I < NINS) {
          const int slot = 64 * I + lane;
          const int row = slot / SPR, ch = min(slot % SPR, SPR - 2);
          lds_dma16(rsq, lq + 1024 * I, row * (int)rq + 16 * ch);
          lds_dma16(rsg, lg + 1024 * I, row * (int)rg + 16 * ch);
        }
      }
    }
  };

  Pos cur = first_from(0);
  if (cur.gi < a.G) {
    fetch(cur);
    dma_tile(cur, 0);
  }
  int buf = 0;
  while (cur.gi < a.G) {
    const int q0 = tile_q0(cur);
    const bool full = cur.t / mq < cur.nfull;
    float slope2 = 0.0f;
    if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
      slope2 = alibi_slope(a.slopes, hk * a.G + cur.gi, a.Hq) * kLog2e;
    // this tile's loads (LDS and registers) have landed; after the barrier
    // every wave has them and is done with the previous tile, whose buffer
    // the next tile's loads then fill
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    sQ = dyn_lds + buf * 2 * kBlock * LDR;
    sG = sQ + kBlock * LDR;
    commit(q0);
    const Pos nxt = next_pos(cur);
    if (nxt.gi < a.G) {
      fetch(nxt);
      dma_tile(nxt, buf ^ 1);
    }
    __syncthreads();  // the tile's LSE, Delta and document ids
    if (full && q0 + kBlock <= a.Q_LEN) tile(q0, slope2, std::false_type{});
    else tile(q0, slope2, std::true_type{});
    cur = nxt;
    buf ^= 1;
  }

  if (kvalid) {
    // result register r of lane l: d = 16*dt + 4*(l/16) + r of key l%16
    u16* ok = a.dk + b * a.sdk[0] + hk * a.sdk[1] + (long long)kv * a.sdk[2];
    u16* ov = a.dv + b * a.sdv[0] + hk * a.sdv[1] + (long long)kv * a.sdv[2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      typename E::V4 pk, pv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pk[r] = (T)(acck[dt][r] * a.scale);
        pv[r] = (T)accv[dt][r];
      }
      *reinterpret_cast<typename E::V4*>(ok + 16 * dt + 4 * g4) = pk;
      *reinterpret_cast<typename E::V4*>(ov + 16 * dt + 4 * g4) = pv;
    }
  }
}

// Delta = dO . O per query row from the forward's fp32 O:
// sum_j P_ij dP_ij = dO_i . sum_j P_ij v_j = dO_i . O_i. D / 8 lanes per row,
// each reading 8 consecutive elements (two 16-byte loads of O, one of dO),
// then a butterfly sum over the row's lanes; a 256-thread block takes
// 2048 / D rows.
template <int D, bool F16>
__global__ __launch_bounds__(256) void delta_from_out_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  constexpr int RPB = 256 / LPR;
  const long long rows = (long long)a.B * a.Hq * a.Q_LEN;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int j = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const int qi = (int)(row % a.Q_LEN);
    const long long bh = row / a.Q_LEN;
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const uint4 gv = *reinterpret_cast<const uint4*>(a.dout + b * a.sdo[0] + h * a.sdo[1] +
                                                     (long long)qi * a.sdo[2] + 8 * j);
    const float4 o0 = *reinterpret_cast<const float4*>(a.o32 + row * D + 8 * j);
    const float4 o1 = *reinterpret_cast<const float4*>(a.o32 + row * D + 8 * j + 4);
    typename BElem<F16>::T g[8];
    __builtin_memcpy(g, &gv, 16);
    const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)g[i], o[i], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && j == 0) a.delta[row] = acc;
}

// A kernel's dynamic-LDS limit is raised once per device to the fixed size
// its launches use (above the 64 KiB a launch gets by default); the flag is
// per kernel (one instantiation each), and concurrent first calls set the
// same value.
template <auto Kernel>
hipError_t raise_lds_limit(int bytes) {
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> raised[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < kMaxDevices && raised[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if (dev < kMaxDevices) raised[dev].store(true, std::memory_order_release);
  return hipSuccess;
}

template <int D, int MASK, int SCORE, bool F16>
hipError_t launch_kernels(const BwdArgs& a, hipStream_t stream) {
  const long long nq = (long long)a.B * a.Hq * a.bm.NQB * (a.bm.QBS / kBlock);
  // dQ: two 64-key K / V step buffers; dK/dV: two query-tile buffers (Q, dO)
  constexpr int kDqLds = 2 * 2 * dq_step_keys<D>() * (D + kPad) * 2;
  constexpr int kKvLds = 2 * 2 * kBlock * (D + kPad) * 2;
  hipError_t e;
  if (a.o32) {
    const long long rows = (long long)a.B * a.Hq * a.Q_LEN;
    constexpr int kRowsPerBlock = 256 / (D / 8);
    delta_from_out_kernel<D, F16>
        <<<(unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock), 256, 0, stream>>>(a);
  } else {
    e = raise_lds_limit<&dq_kernel<D, MASK, SCORE, true, F16>>(kDqLds);
    if (e != hipSuccess) return e;
    dq_kernel<D, MASK, SCORE, true, F16><<<(unsigned)nq, kThreads, kDqLds, stream>>>(a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = raise_lds_limit<&dq_kernel<D, MASK, SCORE, false, F16>>(kDqLds);
  if (e != hipSuccess) return e;
  dq_kernel<D, MASK, SCORE, false, F16><<<(unsigned)nq, kThreads, kDqLds, stream>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nk = (long long)a.B * a.Hkv * a.bm.NKB * (a.bm.BS / kBlock);
  e = raise_lds_limit<&dkdv_kernel<D, MASK, SCORE, F16>>(kKvLds);
  if (e != hipSuccess) return e;
  dkdv_kernel<D, MASK, SCORE, F16><<<(unsigned)nk, 64 * kKvWaves, kKvLds, stream>>>(a);
  return hipGetLastError();
}

template <int D, int MASK, bool F16>
hipError_t dispatch_score(const BwdArgs& a, int score, hipStream_t stream) {
  switch (score) {
    case SCORE_NONE: return launch_kernels<D, MASK, SCORE_NONE, F16>(a, stream);
    case SCORE_ALIBI: return launch_kernels<D, MASK, SCORE_ALIBI, F16>(a, stream);
    case SCORE_SOFTCAP: return launch_kernels<D, MASK, SCORE_SOFTCAP, F16>(a, stream);
    default: return launch_kernels<D, MASK, SCORE_SOFTCAP_ALIBI, F16>(a, stream);
  }
}

template <int D, bool F16>
hipError_t dispatch_mask(const BwdArgs& a, int mask, int score, hipStream_t stream) {
  switch (mask) {
    case MASK_NOOP: return dispatch_score<D, MASK_NOOP, F16>(a, score, stream);
    case MASK_CAUSAL: return dispatch_score<D, MASK_CAUSAL, F16>(a, score, stream);
    case MASK_SLIDING_SINK: return dispatch_score<D, MASK_SLIDING_SINK, F16>(a, score, stream);
    case MASK_PREFIX_LM: return dispatch_score<D, MASK_PREFIX_LM, F16>(a, score, stream);
    case MASK_COMPOSITE: return dispatch_score<D, MASK_COMPOSITE, F16>(a, score, stream);
    default: return dispatch_score<D, MASK_DOCUMENT, F16>(a, score, stream);
  }
}

template <bool F16>
hipError_t launch_elem(const BwdLaunch& L, hipStream_t stream) {
  BwdArgs a;
  a.q = static_cast<const u16*>(L.q);
  a.k = static_cast<const u16*>(L.k);
  a.v = static_cast<const u16*>(L.v);
  a.dout = static_cast<const u16*>(L.dout);
  a.lse = L.lse;
  a.delta = L.delta;
  a.o32 = L.o32;
  a.dq = static_cast<u16*>(L.dq);
  a.dk = static_cast<u16*>(L.dk);
  a.dv = static_cast<u16*>(L.dv);
  for (int i = 0; i < 3; ++i) {
    a.sq[i] = L.sq[i];
    a.sk[i] = L.sk[i];
    a.sv[i] = L.sv[i];
    a.sdo[i] = L.sdo[i];
    a.sdq[i] = L.sdq[i];
    a.sdk[i] = L.sdk[i];
    a.sdv[i] = L.sdv[i];
  }
  a.B = L.B;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.G = L.Hq / L.Hkv;
  a.Q_LEN = L.Q_LEN;
  a.KV_LEN = L.KV_LEN;
  a.mp = L.mp;
  a.scale = L.scale;
  a.c_scale = L.scale * kLog2e;
  a.c_cap = L.softcap > 0.0f ? 2.0f * L.scale * kLog2e / L.softcap : 0.0f;
  a.cap2 = L.softcap * kLog2e;
  a.slopes = L.slopes;
  a.bm = L.bm;
  a.q_num = L.q_num;
  a.q_idx = L.q_idx;
  a.fq_num = L.full_q_num;
  a.fq_idx = L.full_q_idx;
  if (L.D == 64) return dispatch_mask<64, F16>(a, L.mask_kind, L.score_kind, stream);
  return dispatch_mask<128, F16>(a, L.mask_kind, L.score_kind, stream);
}

}  // namespace

#if FA_BWD_F16
hipError_t launch_bwd_f16(const BwdLaunch& L, hipStream_t stream) {
  return launch_elem<true>(L, stream);
}
#else
hipError_t launch_bwd_bf16(const BwdLaunch& L, hipStream_t stream) {
  return launch_elem<false>(L, stream);
}
#endif

}  // namespace fa
