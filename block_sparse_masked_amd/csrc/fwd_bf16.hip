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
// tile); wave w owns query rows [32w, 32w + 32) of the tile. Both products
// use v_mfma_f32_32x32x16_bf16:
//   S^T = K . Q^T   (A = K tile from LDS, B = Q^T held in registers)
//   O^T += V^T . P^T (A = V^T gathered from LDS, B = P^T from registers)
// With the transposed formulation the MFMA result's lane index is the query
// column, so every lane holds scores of one query row (its half of the keys)
// and the row max / sum need one exchange with the partner lane (lane ^ 32);
// the P^T operand is the score accumulator converted in place, and the O^T
// accumulator is rescaled per lane.
//
// MFMA 32x32 result layout: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32. An operand register slot t of
// lane l holds k = 8*(l/32) + t for both A and B; only that A and B agree on
// the k slot matters, so the key order inside the P.V contraction follows
// the S result layout directly.
#include "common.hpp"
#include "fwd_common.hpp"
#include "launch.hpp"

namespace fa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;

constexpr int kThreads = 256;

struct FwdArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  long long sq0, sq1, sq2, sk0, sk1, sk2, sv0, sv1, sv2, so0, so1, so2;
  int B, Hq, Hkv, G, Q_LEN, KV_LEN;
  MaskParams mp;
  float c_scale, c_cap, cap2;
  const float* slopes;
  BlockMaskView bm;
};

// 16-byte chunk swizzle of a [128][D] bf16 tile in LDS: spreads the rows a
// 16-lane phase reads or writes over all banks.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  if constexpr (D == 128) {
    return col ^ (row & 15);
  } else {
    return col ^ ((row >> 1) & 7);
  }
}

// V tile swizzle: the transposed reads take 4 consecutive rows x 32 bytes
// per 16-lane group; XOR-ing the chunk with 2*(row%4) puts those 8 half-chunks
// in distinct banks. Writes of one row's 16-byte chunks stay conflict-free.
__device__ __forceinline__ int swz_v(int row, int col) { return col ^ ((row & 3) << 1); }

template <int D, bool IS_V>
__device__ __forceinline__ void load_tile(u16* lds, const u16* g, long long row_stride, int kv0,
                                          int kv_len) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int N = kBlock * CPR / kThreads;
  uint4 buf[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c / CPR;
    const int col = c % CPR;
    if (kv0 + row < kv_len) {
      buf[i] = *reinterpret_cast<const uint4*>(g + (long long)(kv0 + row) * row_stride + col * 8);
    } else {
      buf[i] = make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c / CPR;
    const int col = c % CPR;
    const int pcol = IS_V ? swz_v(row, col) : swz<D>(row, col);
    *reinterpret_cast<uint4*>(lds + row * D + pcol * 8) = buf[i];
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

template <int D, int MASK, int SCORE>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  __shared__ __attribute__((aligned(16))) u16 sK[kBlock * D];
  __shared__ __attribute__((aligned(16))) u16 sV[kBlock * D];

  const Item it = decode_item(blockIdx.x, a.bm, a.B, a.Hq);
  const int b = it.b, h = it.h;
  const int hk = h / a.G;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int q = it.qb * kBlock + wave * 32 + l32;
  const bool qvalid = q < a.Q_LEN;
  const int qc = qvalid ? q : a.Q_LEN - 1;
  const int vg = (lane >> 4) & 1;  // 16-lane group within the half wave
  const int vi = lane & 15;        // lane within the 16-lane group

  // Q^T operand fragments: lane holds q row `q`, d = 16*ks + 8*hh + [0, 8)
  bf16x8 qf[KSTEPS];
  {
    const u16* qrow = a.q + b * a.sq0 + h * a.sq1 + (long long)qc * a.sq2;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hh));
  }

  const u16* kbase = a.k + b * a.sk0 + hk * a.sk1;
  const u16* vbase = a.v + b * a.sv0 + hk * a.sv1;
  const int* doc = (MASK == MASK_DOCUMENT) ? a.mp.doc + b * a.mp.doc_bstride : nullptr;

  float slope2 = 0.0f;
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
    slope2 = alibi_slope(a.slopes, h, a.Hq) * kLog2e;

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  float m = -INFINITY;
  float l = 0.0f;

  const long long lrow = (long long)it.mrow * a.bm.NKB;
  const int nfull = a.bm.full_num[it.mrow];
  const int npart = a.bm.kv_num[it.mrow];

  for (int t = 0; t < nfull + npart; ++t) {
    const bool partial = t >= nfull;
    const int kb = partial ? a.bm.kv_idx[lrow + (t - nfull)] : a.bm.full_idx[lrow + t];
    const int kv0 = kb * kBlock;
    __syncthreads();
    load_tile<D, false>(sK, kbase, a.sk2, kv0, a.KV_LEN);
    __builtin_amdgcn_sched_barrier(0);
    load_tile<D, true>(sV, vbase, a.sv2, kv0, a.KV_LEN);
    __syncthreads();

    // S^T = K . Q^T, four 32-key blocks
    f32x16 s[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[blk][r] = 0.0f;
      const int row = 32 * blk + l32;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 af = as_bf16x8(
            *reinterpret_cast<const uint4*>(sK + row * D + swz<D>(row, 2 * ks + hh) * 8));
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], s[blk], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // score_mod, mask (partial tiles, and any tile crossing KV_LEN), max
    const bool bounds = kv0 + kBlock > a.KV_LEN;
    const bool do_mask = partial || bounds;
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * blk + 8 * (r >> 2) + 4 * hh + (r & 3);
        float x = ScoreMod<SCORE>::apply(s[blk][r], a.c_scale, a.c_cap, a.cap2, slope2,
                                         (float)(key - q));
        if (do_mask) {
          const bool ok = key < a.KV_LEN && (partial ? Mask<MASK>::allowed(a.mp, doc, qc, key) : true);
          x = ok ? x : -INFINITY;
        }
        s[blk][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float rs = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[blk][r] - m_use);
        s[blk][r] = p;
        rs += p;
      }
    }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;

    // P^T operand: k-step ks covers keys 16*ks .. 16*ks+15 of the tile,
    // slot t <-> result register 8*(ks%2) + t of block ks/2.
    bf16x8 pf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) pf[ks][t2] = (__bf16)s[ks >> 1][8 * (ks & 1) + t2];

    // O^T += V^T . P^T. The V^T operand (lane row d = 32*db + lane%32, slot t
    // <-> key 16*ks + 8*(t/4) + 4*hh + t%4, the key order of pf) comes from
    // the row-major V tile with two transposing reads: in each 16-lane group
    // lane j supplies the 8-byte piece (row j/4, columns 4*(j%4)..+3) of a
    // 4-key x 16-d block and receives column j of that block.
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x4 part[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const int row = 16 * ks + 8 * ht + 4 * hh + (vi >> 2);
          const int d = 32 * db + 16 * vg + 4 * (vi & 3);
          const u16* src = sV + row * D + swz_v(row, d >> 3) * 8 + (d & 7);
          part[ht] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(src));
        }
        const bf16x8 vf = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // epilogue: O = O_acc / l, LSE = ln(sum) + max
  const float l_tot = l + __shfl_xor(l, 32, 64);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qvalid) {
    u16* orow = a.o + b * a.so0 + h * a.so1 + (long long)q * a.so2;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = (__bf16)(o[db][4 * g + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * hh) = pk;
      }
    }
    if (hh == 0) {
      const float lse = l_tot > 0.0f ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
      a.lse[((long long)b * a.Hq + h) * a.Q_LEN + q] = lse;
    }
  }
}

template <int D, int MASK>
hipError_t dispatch_score(const FwdArgs& args, int score, int grid, hipStream_t stream) {
  switch (score) {
    case SCORE_NONE:
      fwd_bf16_kernel<D, MASK, SCORE_NONE><<<grid, kThreads, 0, stream>>>(args);
      break;
    case SCORE_ALIBI:
      fwd_bf16_kernel<D, MASK, SCORE_ALIBI><<<grid, kThreads, 0, stream>>>(args);
      break;
    case SCORE_SOFTCAP:
      fwd_bf16_kernel<D, MASK, SCORE_SOFTCAP><<<grid, kThreads, 0, stream>>>(args);
      break;
    default:
      fwd_bf16_kernel<D, MASK, SCORE_SOFTCAP_ALIBI><<<grid, kThreads, 0, stream>>>(args);
      break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_mask(const FwdArgs& args, int mask, int score, int grid, hipStream_t stream) {
  switch (mask) {
    case MASK_NOOP:
      return dispatch_score<D, MASK_NOOP>(args, score, grid, stream);
    case MASK_CAUSAL:
      return dispatch_score<D, MASK_CAUSAL>(args, score, grid, stream);
    case MASK_SLIDING_SINK:
      return dispatch_score<D, MASK_SLIDING_SINK>(args, score, grid, stream);
    default:
      return dispatch_score<D, MASK_DOCUMENT>(args, score, grid, stream);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdLaunch& L, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const u16*>(L.q);
  a.k = static_cast<const u16*>(L.k);
  a.v = static_cast<const u16*>(L.v);
  a.o = static_cast<u16*>(L.o);
  a.lse = L.lse;
  a.sq0 = L.sq[0]; a.sq1 = L.sq[1]; a.sq2 = L.sq[2];
  a.sk0 = L.sk[0]; a.sk1 = L.sk[1]; a.sk2 = L.sk[2];
  a.sv0 = L.sv[0]; a.sv1 = L.sv[1]; a.sv2 = L.sv[2];
  a.so0 = L.so[0]; a.so1 = L.so[1]; a.so2 = L.so[2];
  a.B = L.B;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.G = L.Hq / L.Hkv;
  a.Q_LEN = L.Q_LEN;
  a.KV_LEN = L.KV_LEN;
  a.mp = L.mp;
  a.c_scale = L.scale * kLog2e;
  a.c_cap = L.softcap > 0.0f ? 2.0f * L.scale * kLog2e / L.softcap : 0.0f;
  a.cap2 = L.softcap * kLog2e;
  a.slopes = L.slopes;
  a.bm = L.bm;
  const int grid = L.B * L.Hq * L.bm.NQB;
  if (grid == 0) return hipSuccess;
  if (L.D == 128) return dispatch_mask<128>(a, L.mask_kind, L.score_kind, grid, stream);
  return dispatch_mask<64>(a, L.mask_kind, L.score_kind, grid, stream);
}

}  // namespace fa
