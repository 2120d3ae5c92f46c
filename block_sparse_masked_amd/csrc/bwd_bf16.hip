// Block-sparse attention backward, bf16 inputs, fp32 accumulation, gfx950.
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
//                 dO_i . O_i, but O is stored in bf16 and the difference
//                 dP - Delta cancels: taken from the bf16 O, Delta's rounding
//                 reaches tens of percent of some rows' dQ, taken this way
//                 it stays at the fp32 level;
//   dq_kernel     the same walk again for dQ;
//   dkdv_kernel   one workgroup per (b, KV head, KV tile); walks the query
//                 tiles of the backward lists for every query head of the
//                 GQA group, so dK / dV are summed in registers with a fixed
//                 order (deterministic, no atomics).
//
// MFMA layout (v_mfma_f32_32x32x16_bf16): an operand fragment is 8 bf16 per
// lane, lane l holding row/column l%32 and k = 8*(l/32) .. +7; a result is 16
// fp32 per lane, register r holding row 8*(r/4) + 4*(l/32) + r%4 and column
// l%32. The 32x32 score tiles are produced with the key (dQ) or the query
// (dK/dV) on the lane axis, so P and dS pack straight into the B operand of
// the next product, whose A operand is read transposed from LDS
// (ds_read_b64_tr_b16) in the matching row order.
//
// Tiles are staged in LDS as row-major blocks with 8 bf16 of padding per row
// (272-byte rows at D = 128), which spreads both the 16-byte row reads and
// the transposed 8-byte reads over the banks without a swizzle.
#include <cmath>

#include "common.hpp"
#include "fwd_common.hpp"
#include "launch.hpp"

namespace fa {
namespace {

typedef unsigned short u16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // four waves
constexpr int kPad = 8;        // bf16 elements of padding per LDS row

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

__device__ __forceinline__ bf16x8 ld_frag(const u16* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// Transposed operand fragment of a row-major LDS block [row][LDR]: lane row
// d = 32*db + lane%32, slot t <-> block row 16*ks + 8*(t/4) + 4*(lane/32) + t%4.
// Each 16-lane group of a ds_read_b64_tr_b16 supplies the 8-byte pieces (row
// j/4, columns 4*(j%4) .. +3) of a 4-row x 16-column block and lane j gets
// column j of it.
template <int LDR>
__device__ __forceinline__ bf16x8 tr_frag(const u16* blk, int lane, int ks, int db) {
  const int hh = lane >> 5, vg = (lane >> 4) & 1, vi = lane & 15;
  const int row = 16 * ks + 4 * hh + (vi >> 2);
  const int col = 32 * db + 16 * vg + 4 * (vi & 3);
  bf16x4 part[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
    part[ht] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(blk + (row + 8 * ht) * LDR + col));
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// Rows [r0, r0 + 128) of a [len][D] bf16 matrix (row stride `ld` elements)
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
    return kv <= q && dq == dkv;
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

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, h, query tile); wave w owns query rows
// 32w .. 32w+31 of the tile. Per 32-key block: S^T = K.Q^T and dP^T = V.dO^T
// (key rows on the register axis, query on the lane axis), dS^T, then
// dQ^T += K^T . dS^T with K read transposed from LDS. With DELTA the walk
// only sums P dP per query row and writes Delta.
// ---------------------------------------------------------------------------
template <int D, int MASK, int SCORE, bool DELTA>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(BwdArgs a) {
  constexpr int LDR = D + kPad;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) u16 sK[kBlock * LDR];
  __shared__ __attribute__((aligned(16))) u16 sV[kBlock * LDR];
  __shared__ int sdoc[kBlock];

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

  bf16x8 qf[KS], dof[KS];
  {
    const u16* qrow = a.q + b * a.sq[0] + h * a.sq[1] + (long long)qc * a.sq[2];
    const u16* grow = a.dout + b * a.sdo[0] + h * a.sdo[1] + (long long)qc * a.sdo[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = ld_frag(qrow + 16 * ks + 8 * hh);
      dof[ks] = ld_frag(grow + 16 * ks + 8 * hh);
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

  auto tile = [&](int kv0, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll 1
    for (int blk = 0; blk < kBlock / 32; ++blk) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const u16* krow = sK + (32 * blk + l32) * LDR + 8 * hh;
      const u16* vrow = sV + (32 * blk + l32) * LDR + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_frag(krow + 16 * ks), qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_frag(vrow + 16 * ks), dof[ks], dp, 0, 0,
                                                     0);
      }
      bf16x8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 32 * blk + 8 * (r >> 2) + 4 * hh + (r & 3);
        float x, dm;
        logit_and_slope<MASK, SCORE, MASKED>(s[r], q, kv0 + kl, dq_id,
                                             mask_uses_doc(MASK) ? sdoc[kl] : 0, slope2, a,
                                             x, dm);
        const float p = fast_exp2(x - lse2);
        if constexpr (DELTA) psum = fmaf(p, dp[r], psum);
        else dsf[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dlt) * dm);
      }
      if constexpr (!DELTA) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < DB; ++db)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                tr_frag<LDR>(sK, lane, 2 * blk + k2, db), dsf[k2], acc[db], 0, 0, 0);
      }
    }
  };

  for (int t = 0; t < (nfull + npart) * mk; ++t) {
    const int c = t / mk;  // listed tile; its 128-key piece t % mk
    const bool full = c < nfull;
    const int kb = min(max(full ? a.bm.full_idx[lrow + c] : a.bm.kv_idx[lrow + c - nfull], 0),
                       NKB - 1);
    const int kv0 = kb * a.bm.BS + (t - c * mk) * kBlock;
    __syncthreads();  // the previous tile's reads are done
    stage_rows<D, 2>(sK, kbase, a.sk[2], kv0, a.KV_LEN, tid);
    stage_rows<D, 2>(sV, vbase, a.sv[2], kv0, a.KV_LEN, tid);
    if constexpr (mask_uses_doc(MASK)) {
      if (doc_row)
        for (int i = tid; i < kBlock; i += kThreads)
          sdoc[i] = (kv0 + i < a.KV_LEN) ? doc_row[kv0 + i] : -1;
    }
    __syncthreads();
    if (full && kv0 + kBlock <= a.KV_LEN) tile(kv0, std::false_type{});
    else tile(kv0, std::true_type{});
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
        bf16x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = (__bf16)(acc[db][4 * gq + j] * a.scale);
        *reinterpret_cast<bf16x4*>(out + 32 * db + 8 * gq + 4 * hh) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, KV head, KV tile); wave w owns key rows
// 32w .. 32w+31. For every query head of the group and every query tile of
// the backward lists, per 32-query block: S = Q.K^T and dP = dO.V^T (query
// rows on the register axis, key on the lane axis), then dV^T += dO^T . P^T
// and dK^T += Q^T . dS^T with dO and Q read transposed from LDS.
// ---------------------------------------------------------------------------
template <int D, int MASK, int SCORE>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int LDR = D + kPad;
  constexpr int KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) u16 sQ[kBlock * LDR];
  __shared__ __attribute__((aligned(16))) u16 sG[kBlock * LDR];  // dO
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
  const int l32 = lane & 31, hh = lane >> 5;
  const int kv = kb * kBlock + wave * 32 + l32;
  const bool kvalid = kv < a.KV_LEN;
  const int kvc = kvalid ? kv : a.KV_LEN - 1;

  bf16x8 kf[KS], vf[KS];
  {
    const u16* krow = a.k + b * a.sk[0] + hk * a.sk[1] + (long long)kvc * a.sk[2];
    const u16* vrow = a.v + b * a.sv[0] + hk * a.sv[1] + (long long)kvc * a.sv[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = ld_frag(krow + 16 * ks + 8 * hh);
      vf[ks] = ld_frag(vrow + 16 * ks + 8 * hh);
    }
  }
  const int* doc_row =
      (mask_uses_doc(MASK) && a.mp.doc) ? a.mp.doc + b * a.mp.doc_bstride : nullptr;
  const int dkv_id = doc_row ? doc_row[kvc] : 0;

  f32x16 acck[DB], accv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    acck[i] = f32x16{};
    accv[i] = f32x16{};
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

  // The next tile's Q / dO rows (and LSE, Delta, document ids) are loaded
  // into registers while the current tile computes, then written to LDS.
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int PER = kBlock * CH / kThreads;  // chunks per thread
  uint4 pq[PER], pg[PER];
  float pl = 0.0f, pd = 0.0f;
  int pdoc = 0;
  auto fetch = [&](const Pos& p) __attribute__((always_inline)) {
    const int h = hk * a.G + p.gi;
    const int q0 = tile_q0(p);
    const u16* qbase = a.q + b * a.sq[0] + h * a.sq[1];
    const u16* gbase = a.dout + b * a.sdo[0] + h * a.sdo[1];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kThreads;
      const int rr = min(q0 + c / CH, a.Q_LEN - 1);
      pq[i] = *reinterpret_cast<const uint4*>(qbase + (long long)rr * a.sq[2] + (c % CH) * 8);
      pg[i] = *reinterpret_cast<const uint4*>(gbase + (long long)rr * a.sdo[2] + (c % CH) * 8);
    }
    if (tid < kBlock) {
      const long long lrow = ((long long)b * a.Hq + h) * a.Q_LEN + min(q0 + tid, a.Q_LEN - 1);
      pl = a.lse[lrow];
      pd = a.delta[lrow];
      if constexpr (mask_uses_doc(MASK))
        if (doc_row) pdoc = doc_row[min(q0 + tid, a.Q_LEN - 1)];
    }
  };
  auto commit = [&](int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / CH;
      const bool in = q0 + r < a.Q_LEN;
      uint4 wq = pq[i], wg = pg[i];
      wq.x = in ? wq.x : 0u; wq.y = in ? wq.y : 0u; wq.z = in ? wq.z : 0u; wq.w = in ? wq.w : 0u;
      wg.x = in ? wg.x : 0u; wg.y = in ? wg.y : 0u; wg.z = in ? wg.z : 0u; wg.w = in ? wg.w : 0u;
      *reinterpret_cast<uint4*>(sQ + r * LDR + (c % CH) * 8) = wq;
      *reinterpret_cast<uint4*>(sG + r * LDR + (c % CH) * 8) = wg;
    }
    if (tid < kBlock) {
      const bool in = q0 + tid < a.Q_LEN;
      slse[tid] = in ? lse_base2(pl) : INFINITY;
      sdel[tid] = in ? pd : 0.0f;
      if constexpr (mask_uses_doc(MASK)) sdoc[tid] = in ? pdoc : -2;
    }
  };

  auto tile = [&](int q0, float slope2, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll 1
    for (int qs = 0; qs < kBlock / 32; ++qs) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const u16* qrow = sQ + (32 * qs + l32) * LDR + 8 * hh;
      const u16* grow = sG + (32 * qs + l32) * LDR + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_frag(qrow + 16 * ks), kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_frag(grow + 16 * ks), vf[ks], dp, 0, 0,
                                                     0);
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql0 = 32 * qs + 8 * g4 + 4 * hh;
        const float4 l4 = *reinterpret_cast<const float4*>(slse + ql0);
        const float4 d4 = *reinterpret_cast<const float4*>(sdel + ql0);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g4 + j;
          const int ql = ql0 + j;
          float x, dm;
          logit_and_slope<MASK, SCORE, MASKED>(s[r], q0 + ql, kv,
                                               mask_uses_doc(MASK) ? sdoc[ql] : 0, dkv_id,
                                               slope2, a, x, dm);
          const float p = fast_exp2(x - lv[j]);
          pf[r >> 3][r & 7] = (__bf16)p;
          dsf[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl[j]) * dm);
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          accv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_frag<LDR>(sG, lane, 2 * qs + k2, db), pf[k2], accv[db], 0, 0, 0);
          acck[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_frag<LDR>(sQ, lane, 2 * qs + k2, db), dsf[k2], acck[db], 0, 0, 0);
        }
    }
  };


  Pos cur = first_from(0);
  if (cur.gi < a.G) fetch(cur);
  while (cur.gi < a.G) {
    const int q0 = tile_q0(cur);
    const bool full = cur.t / mq < cur.nfull;
    float slope2 = 0.0f;
    if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
      slope2 = alibi_slope(a.slopes, hk * a.G + cur.gi, a.Hq) * kLog2e;
    __syncthreads();  // the previous tile's reads are done
    commit(q0);
    __syncthreads();
    const Pos nxt = next_pos(cur);
    if (nxt.gi < a.G) fetch(nxt);
    if (full && q0 + kBlock <= a.Q_LEN) tile(q0, slope2, std::false_type{});
    else tile(q0, slope2, std::true_type{});
    cur = nxt;
  }

  if (kvalid) {
    u16* ok = a.dk + b * a.sdk[0] + hk * a.sdk[1] + (long long)kv * a.sdk[2];
    u16* ov = a.dv + b * a.sdv[0] + hk * a.sdv[1] + (long long)kv * a.sdv[2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        bf16x4 pk, pv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pk[j] = (__bf16)(acck[db][4 * gq + j] * a.scale);
          pv[j] = (__bf16)accv[db][4 * gq + j];
        }
        *reinterpret_cast<bf16x4*>(ok + 32 * db + 8 * gq + 4 * hh) = pk;
        *reinterpret_cast<bf16x4*>(ov + 32 * db + 8 * gq + 4 * hh) = pv;
      }
  }
}

// Delta = dO . O per query row from the forward's fp32 O (one wave per row):
// sum_j P_ij dP_ij = dO_i . sum_j P_ij v_j = dO_i . O_i.
template <int D>
__global__ __launch_bounds__(256) void delta_from_out_kernel(BwdArgs a) {
  constexpr int PER = D / 64;
  const long long rows = (long long)a.B * a.Hq * a.Q_LEN;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int qi = (int)(row % a.Q_LEN);
  const long long bh = row / a.Q_LEN;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const u16* g = a.dout + b * a.sdo[0] + h * a.sdo[1] + (long long)qi * a.sdo[2] + lane * PER;
  const float* o = a.o32 + row * D + lane * PER;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    __bf16 gv;
    __builtin_memcpy(&gv, g + i, 2);
    acc = fmaf((float)gv, o[i], acc);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) a.delta[row] = acc;
}

template <int D, int MASK, int SCORE>
hipError_t launch_kernels(const BwdArgs& a, hipStream_t stream) {
  const long long nq = (long long)a.B * a.Hq * a.bm.NQB * (a.bm.QBS / kBlock);
  if (a.o32) {
    const long long rows = (long long)a.B * a.Hq * a.Q_LEN;
    delta_from_out_kernel<D><<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(a);
  } else {
    dq_kernel<D, MASK, SCORE, true><<<(unsigned)nq, kThreads, 0, stream>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dq_kernel<D, MASK, SCORE, false><<<(unsigned)nq, kThreads, 0, stream>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long nk = (long long)a.B * a.Hkv * a.bm.NKB * (a.bm.BS / kBlock);
  dkdv_kernel<D, MASK, SCORE><<<(unsigned)nk, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int MASK>
hipError_t dispatch_score(const BwdArgs& a, int score, hipStream_t stream) {
  switch (score) {
    case SCORE_NONE: return launch_kernels<D, MASK, SCORE_NONE>(a, stream);
    case SCORE_ALIBI: return launch_kernels<D, MASK, SCORE_ALIBI>(a, stream);
    case SCORE_SOFTCAP: return launch_kernels<D, MASK, SCORE_SOFTCAP>(a, stream);
    default: return launch_kernels<D, MASK, SCORE_SOFTCAP_ALIBI>(a, stream);
  }
}

template <int D>
hipError_t dispatch_mask(const BwdArgs& a, int mask, int score, hipStream_t stream) {
  switch (mask) {
    case MASK_NOOP: return dispatch_score<D, MASK_NOOP>(a, score, stream);
    case MASK_CAUSAL: return dispatch_score<D, MASK_CAUSAL>(a, score, stream);
    case MASK_SLIDING_SINK: return dispatch_score<D, MASK_SLIDING_SINK>(a, score, stream);
    case MASK_PREFIX_LM: return dispatch_score<D, MASK_PREFIX_LM>(a, score, stream);
    case MASK_COMPOSITE: return dispatch_score<D, MASK_COMPOSITE>(a, score, stream);
    default: return dispatch_score<D, MASK_DOCUMENT>(a, score, stream);
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdLaunch& L, hipStream_t stream) {
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
  if (L.D == 64) return dispatch_mask<64>(a, L.mask_kind, L.score_kind, stream);
  return dispatch_mask<128>(a, L.mask_kind, L.score_kind, stream);
}

}  // namespace fa
