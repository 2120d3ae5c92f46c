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
// tile); wave w owns query rows [32w, 32w + 32). Both products use
// v_mfma_f32_32x32x16_bf16:
//   S^T = K . Q^T    (A = K tile from LDS, B = Q^T held in registers)
//   O^T += V^T . P^T (A = V^T read transposed from LDS, B = P^T in registers)
// The MFMA result's lane index is the query column, so each lane holds the
// scores of one query row (half of the tile's keys); the row max needs one
// exchange with lane ^ 32, the P^T operand is the converted score registers
// and the O^T accumulator is rescaled per lane.
//
// MFMA 32x32 result layout: register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32. An operand register slot t of
// lane l holds k = 8*(l/32) + t for both A and B, so the key order inside the
// P.V contraction follows the S result layout directly.
//
// Pipeline per KV tile j (K and V double-buffered in LDS, filled with direct
// global->LDS loads):
//   issue loads of V[j+1] and K[j+2]
//   S[j+1] = K[j+1] . Q^T on the matrix cores, overlapped with the softmax of
//   S[j] on the vector ALUs; then O += V[j] . P[j]
//   wait for the loads, barrier
// Full tiles take a path with no mask code. The running max is applied
// lazily: O and the row sum are rescaled only when a row's max grows by more
// than 2^8 (exp2 units), which leaves the result unchanged (any reference
// point gives the same normalised sums) while skipping most rescales.
#include "common.hpp"
#include "fwd_common.hpp"
#include "launch.hpp"

namespace fa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.0f;  // exp2 units: p <= 256 between rescales

struct FwdArgs {
  const u16* q;
  const u16* k;
  const u16* v;
  u16* o;
  float* lse;
  long long sq0, sq1, sq2, sk0, sk1, sk2, sv0, sv1, sv2, so0, so1, so2;
  int B, Hq, Hkv, G, Q_LEN, KV_LEN;
  int xcd_round;  // > 0: items per schedule round, remapped so KV groups share an XCD
  int doc_len;
  MaskParams mp;
  float c_scale, c_cap, cap2;
  const float* slopes;
  BlockMaskView bm;
};

// 16-byte chunk swizzle of a K tile [128][D] in LDS: the 16 rows a
// 16-lane phase of a fragment read touches land in distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  if constexpr (D == 128) {
    return col ^ (row & 15);
  } else {
    return col ^ ((row >> 1) & 7);
  }
}

// V tile swizzle: a transposed read takes 4 consecutive rows x 32 bytes per
// 16-lane group; XOR-ing the chunk with 2*(row%4) puts those 8 half-chunks in
// distinct banks.
__device__ __forceinline__ int swz_v(int row, int col) { return col ^ ((row & 3) << 1); }

// Direct global->LDS loads of one [128][D] bf16 tile through a buffer
// resource. Each wave-wide load fills one contiguous KiB of LDS (lane l
// writes bytes [16 l, 16 l + 16)), so each lane fetches the global chunk
// whose swizzled home is that slot; its byte offset inside the tile is fixed
// and computed once. Per tile only the resource base moves, and its size ends
// at the last key row, so rows past kv_len read as zero (their scores are
// masked: a tile crossing kv_len always takes the masked path).
template <int D, bool IS_V>
struct TileLoader {
  static constexpr int CPR = D / 8;
  static constexpr int ROWS_PER_KB = 1024 / (2 * D);
  static constexpr int KB_PER_WAVE = (kBlock / ROWS_PER_KB) / 4;
  int voff[KB_PER_WAVE];
  int lds_off;  // element offset of this wave's first KiB inside a tile

  __device__ void init(int wave, int lane, long long stride) {
    const int r_in = lane / CPR;
    const int pch = lane % CPR;
#pragma unroll
    for (int i = 0; i < KB_PER_WAVE; ++i) {
      const int row = (wave * KB_PER_WAVE + i) * ROWS_PER_KB + r_in;
      const int col = IS_V ? swz_v(row, pch) : swz<D>(row, pch);
      voff[i] = (int)(row * stride * 2) + col * 16;
    }
    lds_off = wave * KB_PER_WAVE * 512;
  }

  __device__ __forceinline__ void issue(u16* lds, const u16* g, long long stride, int kv0,
                                        int kv_len) const {
    // (device pass only: the host pass of this compiler drops the kernel
    // stubs of functions that name the buffer-resource type)
#if defined(__HIP_DEVICE_COMPILE__)
    const long long bytes = (long long)(kv_len - kv0) * stride * 2;
    const int nrec = bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes;
    __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(g + (long long)kv0 * stride), (short)0, nrec,
                                          0x00020000);
#pragma unroll
    for (int i = 0; i < KB_PER_WAVE; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(lds + lds_off + i * 512), 16, voff[i],
                                               0, 0, 0);
#endif
  }
};

__device__ __forceinline__ void wait_loads_and_sync() {
  // vmcnt(0), expcnt/lgkmcnt unconstrained, then the workgroup barrier
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
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
  float slope2;
  int dq;  // document id of this lane's query row (document mask)
  int kofs[D / 16];  // K fragment (row l32 of block 0, k-step ks)
  int vofs[D / 32];  // V transposed-read piece (k-step 0, half 0, d-block db)

  __device__ void init_offsets() {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kofs[ks] = l32 * D + swz<D>(l32, 2 * ks + hh) * 8;
    const int row = 4 * hh + (vi >> 2);  // + 16*ks + 8*half: multiples of 4 leave row % 4 alone
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = 32 * db + 16 * vg + 4 * (vi & 3);
      vofs[db] = row * D + swz_v(row, d >> 3) * 8 + (d & 7);
    }
  }
};

// S^T = K . Q^T for the four 32-key blocks of a tile.
template <int D>
__device__ __forceinline__ void compute_s(f32x16 (&s)[4], const u16* sK, const bf16x8 (&qf)[D / 16],
                                          const Lane<D>& ln) {
#pragma unroll
  for (int blk = 0; blk < 4; ++blk)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[blk][r] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      // rows 32*blk + l32: block offsets keep row % 16 (and (row/2) % 8)
      const bf16x8 af =
          as_bf16x8(*reinterpret_cast<const uint4*>(sK + ln.kofs[ks] + 32 * blk * D));
      s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], s[blk], 0, 0, 0);
    }
  }
  // scores feed the vector ALUs: keep them in VGPRs
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) asm volatile("" : "+v"(s[blk]));
#endif
}

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x0002;
constexpr int kSgMfma = 0x0008;
constexpr int kSgDsRead = 0x0100;

// Row max across the two lanes that hold one query row (lane, lane ^ 32).
__device__ __forceinline__ float pair_max(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                   false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// O^T += V^T . P^T for one tile (32 MFMAs). The V^T fragment (lane row
// d = 32*db + lane%32, slot t <-> key 16*ks + 8*(t/4) + 4*hh + t%4, the key
// order of pf) comes from the row-major V tile with two transposing reads: in
// each 16-lane group lane j supplies the 8-byte piece (row j/4, columns
// 4*(j%4)..+3) of a 4-key x 16-d block and receives column j of that block.
template <int D>
__device__ __forceinline__ void pv(f32x16 (&o)[D / 32], const bf16x8 (&pf)[8], const u16* sV,
                                   const Lane<D>& ln) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      bf16x4 part[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const u16* src = sV + ln.vofs[db] + (16 * ks + 8 * ht) * D;
        part[ht] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(src));
      }
      const bf16x8 vf = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[db], 0, 0, 0);
    }
  }
  // keep O in the accumulation registers (one workgroup per CU: 512
  // registers per lane, the score and probability registers stay in VGPRs)
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int db = 0; db < D / 32; ++db) asm volatile("" : "+a"(o[db]));
#endif
}

// Score modification of tile kv0 in place (base-2 logits) and the lane's max.
// Without a score_mod the raw scores stay in place: scale > 0, so the max of
// the raw scores times scale*log2(e) is the logit max, and the scale is
// folded into the exponent's FMA.
template <int D, int SCORE>
__device__ __forceinline__ float logits(f32x16 (&s)[4], int kv0, const FwdArgs& a,
                                        const Lane<D>& ln) {
  float mx = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (SCORE != SCORE_NONE) {
        const int key = kv0 + 32 * blk + 8 * (r >> 2) + 4 * ln.hh + (r & 3);
        s[blk][r] = ScoreMod<SCORE>::apply(s[blk][r], a.c_scale, a.c_cap, a.cap2, ln.slope2,
                                           (float)(key - ln.q));
      }
      mx = fmaxf(mx, s[blk][r]);
    }
  }
  return mx;
}

// mask_mod on a partial tile (and the key bound), in place; returns the new
// max. For the document mask the tile's 128 key document ids are in LDS.
template <int D, int MASK>
__device__ __forceinline__ float apply_mask(f32x16 (&s)[4], int kv0, const int* tile_doc,
                                            const FwdArgs& a, const Lane<D>& ln) {
  float mx = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      int4 dk = make_int4(0, 0, 0, 0);
      if constexpr (MASK == MASK_DOCUMENT)
        dk = *reinterpret_cast<const int4*>(tile_doc + 32 * blk + 8 * g + 4 * ln.hh);
      const int dks[4] = {dk.x, dk.y, dk.z, dk.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g + j;
        const int key = kv0 + 32 * blk + 8 * g + 4 * ln.hh + j;
        bool ok = key < a.KV_LEN;
        if constexpr (MASK == MASK_DOCUMENT) {
          ok = ok && key <= ln.qc && dks[j] == ln.dq;
        } else {
          ok = ok && Mask<MASK>::allowed(a.mp, nullptr, ln.qc, key);
        }
        s[blk][r] = ok ? s[blk][r] : -INFINITY;
        mx = fmaxf(mx, s[blk][r]);
      }
    }
  }
  return mx;
}

// One tile of the pipeline:
//   phase 1: O += V[j-1] . P[j-1] interleaved with the logits and row max
//            of S[j] (for j = 0, P is zero and the V buffer is zero-filled);
//   lazy rescale of O and l when a row max moved up by more than 2^8;
//   phase 2: S[j+1] = K[j+1] . Q^T interleaved with exp, row sum and the
//            bf16 conversion of S[j] into P[j].
template <int D, int MASK, int SCORE>
__device__ __forceinline__ void step(f32x16 (&s)[4], f32x16 (&s_next)[4], f32x16 (&o)[D / 32],
                                     bf16x8 (&pf)[8], float& m_ref, float& l,
                                     const bf16x8 (&qf)[D / 16], const u16* sK_next,
                                     const u16* sV_prev, int kv0, bool masked,
                                     const int* tile_doc, const FwdArgs& a, const Lane<D>& ln) {
  constexpr int DB = D / 32;
  constexpr int NMFMA_PV = 8 * DB;
  constexpr int NMFMA_S = 4 * (D / 16);
  // phase 1: P.V of the previous tile || logits and max of this tile
  pv<D>(o, pf, sV_prev, ln);
  float mx = logits<D, SCORE>(s, kv0, a, ln);
  // transposed V reads run two MFMAs ahead of their products
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
  for (int i = 0; i < NMFMA_PV; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if (i + 2 < NMFMA_PV) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSgValu, SCORE == SCORE_NONE ? 2 : 6, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (masked) mx = apply_mask<D, MASK>(s, kv0, tile_doc, a, ln);
  mx = pair_max(mx);
  if constexpr (SCORE == SCORE_NONE) mx *= a.c_scale;

  // lazy rescale when some row's max exceeds its reference by 2^8
  if (__any(mx > m_ref + kRescaleSlack)) {
    const float m_new = fmaxf(m_ref, mx);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_ref - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
    m_ref = m_new;
  }
  const float m_use = (m_ref == -INFINITY) ? 0.0f : m_ref;
  __builtin_amdgcn_sched_barrier(0);

  // phase 2: S of the next tile || exponentials, row sum, bf16 P
  compute_s<D>(s_next, sK_next, qf, ln);
  float rs = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float x = s[ks >> 1][8 * (ks & 1) + t];
      float p;
      if constexpr (SCORE == SCORE_NONE) {
        p = fast_exp2(fmaf(x, a.c_scale, -m_use));
      } else {
        p = fast_exp2(x - m_use);
      }
      rs += p;
      pf[ks][t] = (__bf16)p;
    }
  }
  l += rs;
  // K fragment reads run two MFMAs ahead of their products
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 1);
#pragma unroll
  for (int i = 0; i < NMFMA_S; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 1);
    if (i + 2 < NMFMA_S) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 1);
    __builtin_amdgcn_sched_group_barrier(kSgValu, 224 / NMFMA_S, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, int MASK, int SCORE>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int TILE = kBlock * D;  // elements of one K or V tile
  // LDS: K and V tiles double-buffered as separate arrays (so the compiler
  // can tell the buffer being filled from the one being read and does not
  // wait for in-flight loads before LDS reads), two 128-entry document-id
  // buffers, and the item's tile list (NKB ints, dynamic)
  __shared__ __attribute__((aligned(16))) u16 sK0[TILE];
  __shared__ __attribute__((aligned(16))) u16 sK1[TILE];
  __shared__ __attribute__((aligned(16))) u16 sV0[TILE];
  __shared__ __attribute__((aligned(16))) u16 sV1[TILE];
  __shared__ __attribute__((aligned(16))) int docbuf[2 * 128];
  extern __shared__ __attribute__((aligned(16))) int tlist[];

  // dispatch order -> item; rounds of equal tile count are remapped so the
  // heads sharing a KV head run on one XCD (workgroups go round-robin to XCDs)
  int x = blockIdx.x;
  if (a.xcd_round > 0) {
    const int R = a.xcd_round;
    const int r = x / R, u = x - r * R;
    x = r * R + (u & 7) * (R >> 3) + (u >> 3);
  }
  const Item it = decode_item(x, a.bm, a.B, a.Hq);
  const int b = it.b, h = it.h;
  const int hk = h / a.G;
  const int wave = threadIdx.x >> 6;
  Lane<D> ln;
  ln.lane = threadIdx.x & 63;
  ln.l32 = ln.lane & 31;
  ln.hh = ln.lane >> 5;
  ln.vg = (ln.lane >> 4) & 1;
  ln.vi = ln.lane & 15;
  ln.q = it.qb * kBlock + wave * 32 + ln.l32;
  const bool qvalid = ln.q < a.Q_LEN;
  ln.qc = qvalid ? ln.q : a.Q_LEN - 1;
  const int* doc_row = (MASK == MASK_DOCUMENT) ? a.mp.doc + b * a.mp.doc_bstride : nullptr;
  ln.dq = (MASK == MASK_DOCUMENT) ? doc_row[ln.qc] : 0;
  ln.init_offsets();
  ln.slope2 = 0.0f;
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
    ln.slope2 = alibi_slope(a.slopes, h, a.Hq) * kLog2e;

  const u16* kbase = a.k + b * a.sk0 + hk * a.sk1;
  const u16* vbase = a.v + b * a.sv0 + hk * a.sv1;
  TileLoader<D, false> kload;
  TileLoader<D, true> vload;
  kload.init(wave, ln.lane, a.sk2);
  vload.init(wave, ln.lane, a.sv2);
  const long long lrow = (long long)it.mrow * a.bm.NKB;
  // counts are clamped to the list length so a malformed BlockMask cannot
  // index past the staged list
  const int nfull = min(a.bm.full_num[it.mrow], a.bm.NKB);
  const int n = min(nfull + a.bm.kv_num[it.mrow], a.bm.NKB);
  // the item's tiles, full then partial, staged in LDS once
  for (int t = threadIdx.x; t < n; t += kThreads)
    tlist[t] = t < nfull ? a.bm.full_idx[lrow + t] : a.bm.kv_idx[lrow + (t - nfull)];
  auto tile_kv0 = [&](int t) { return kBlock * __builtin_amdgcn_readfirstlane(tlist[t]); };
  // document ids of a tile's keys -> docbuf[i] (rows past KV_LEN read as 0)
  auto issue_doc = [&](int* dst, int kv0) {
    if constexpr (MASK == MASK_DOCUMENT) {
#if defined(__HIP_DEVICE_COMPILE__)
      if (wave == 0) {
        const int nrec = 4 * (min(a.KV_LEN, a.doc_len) - kv0);
        __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(doc_row + kv0), (short)0, nrec > 0 ? nrec : 0, 0x00020000);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(dst + 64 * c), 4,
                                                   4 * ln.lane + 256 * c, 0, 0, 0);
      }
#endif
    }
  };

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.0f;
  float m_ref = -INFINITY;
  float l = 0.0f;

  __syncthreads();  // tile list visible
  if (n > 0) {
    // prologue: K[0] -> K buffer 0, K[1] -> K buffer 1, Q^T fragments; S[0]
    int kv0 = tile_kv0(0);
    issue_doc(docbuf, kv0);
    kload.issue(sK0, kbase, a.sk2, kv0, a.KV_LEN);
    if (n > 1) kload.issue(sK1, kbase, a.sk2, tile_kv0(1), a.KV_LEN);
    bf16x8 qf[KSTEPS];
    {
      const u16* qrow = a.q + b * a.sq0 + h * a.sq1 + (long long)ln.qc * a.sq2;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * ln.hh));
    }
    // V buffer 1 is read by the first tile's (empty) P.V: zero it, P = 0
    for (int i = threadIdx.x; i < TILE / 8; i += kThreads)
      reinterpret_cast<uint4*>(sV1)[i] = make_uint4(0, 0, 0, 0);
    wait_loads_and_sync();
    f32x16 s[4], s2[4];
    bf16x8 pf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int t = 0; t < 8; ++t) pf[ks][t] = (__bf16)0.0f;
    compute_s<D>(s, sK0, qf, ln);

    // Tile j: at entry, K[j+1] and V[j-1] are resident; issue V[j] into V
    // buffer j%2 (it held V[j-2]) and K[j+2] into K buffer j%2 (it held K[j]).
    // The next tile's S is always computed; on the last tile it reads a stale
    // buffer and is discarded (hidden under that tile's softmax).
    // even tiles: load into the *0 buffers, read K1 / V1; odd tiles: the
    // other way round (two tiles per trip so every buffer is fixed)
    auto stage = [&](int j, f32x16(&cur)[4], f32x16(&nxt)[4], u16* kw, u16* vw, const u16* kr,
                     const u16* vr, int* dw, const int* dr) {
      const int kv_next = tile_kv0(j + 1 < n ? j + 1 : j);
      const int kv_after = tile_kv0(j + 2 < n ? j + 2 : j);
      vload.issue(vw, vbase, a.sv2, kv0, a.KV_LEN);
      if (j + 2 < n) kload.issue(kw, kbase, a.sk2, kv_after, a.KV_LEN);
      if (j + 1 < n) issue_doc(dw, kv_next);
      const bool masked = (j >= nfull) || (kv0 + kBlock > a.KV_LEN);
      step<D, MASK, SCORE>(cur, nxt, o, pf, m_ref, l, qf, kr, vr, kv0, masked, dr, a, ln);
      kv0 = kv_next;
      wait_loads_and_sync();
    };
    for (int j = 0; j < n; j += 2) {
      stage(j, s, s2, sK0, sV0, sK1, sV1, docbuf + 128, docbuf);
      if (j + 1 >= n) break;
      stage(j + 1, s2, s, sK1, sV1, sK0, sV0, docbuf, docbuf + 128);
    }
    const u16* vlast = ((n - 1) & 1) ? sV1 : sV0;
    // the last tile's P . V
    pv<D>(o, pf, vlast, ln);
  }

  // epilogue: O = O_acc / l, LSE = ln(sum) + max
  const float l_tot = l + __shfl_xor(l, 32, 64);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qvalid) {
    u16* orow = a.o + b * a.so0 + h * a.so1 + (long long)ln.q * a.so2;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = (__bf16)(o[db][4 * g + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * ln.hh) = pk;
      }
    }
    if (ln.hh == 0) {
      const float lse = l_tot > 0.0f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
      a.lse[((long long)b * a.Hq + h) * a.Q_LEN + ln.q] = lse;
    }
  }
}

template <int D, int MASK, int SCORE>
hipError_t launch_one(const FwdArgs& args, int grid, hipStream_t stream) {
  const int lds = 4 * ((args.bm.NKB + 3) & ~3);
  static int attr_bytes = 0;
  if (lds > attr_bytes) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&fwd_bf16_kernel<D, MASK, SCORE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_bytes = lds;
  }
  fwd_bf16_kernel<D, MASK, SCORE><<<grid, kThreads, lds, stream>>>(args);
  return hipGetLastError();
}

template <int D, int MASK>
hipError_t dispatch_score(const FwdArgs& args, int score, int grid, hipStream_t stream) {
  switch (score) {
    case SCORE_NONE:
      return launch_one<D, MASK, SCORE_NONE>(args, grid, stream);
    case SCORE_ALIBI:
      return launch_one<D, MASK, SCORE_ALIBI>(args, grid, stream);
    case SCORE_SOFTCAP:
      return launch_one<D, MASK, SCORE_SOFTCAP>(args, grid, stream);
    default:
      return launch_one<D, MASK, SCORE_SOFTCAP_ALIBI>(args, grid, stream);
  }
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

int fwd_bf16_lds_bytes(int D, int NKB) {
  return 4 * kBlock * D * 2 + 4 * ((NKB + 3) & ~3) + 2 * 128 * 4;
}

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
  a.doc_len = L.doc_len;
  a.c_scale = L.scale * kLog2e;
  a.c_cap = L.softcap > 0.0f ? 2.0f * L.scale * kLog2e / L.softcap : 0.0f;
  a.cap2 = L.softcap * kLog2e;
  a.slopes = L.slopes;
  a.bm = L.bm;
  // XCD-aware order: with the mask broadcast over batch and heads every
  // schedule round holds the B*Hq rows of one query tile; split each round
  // into 8 contiguous chunks of whole KV groups, one per XCD.
  const int R = L.B * L.Hq;
  a.xcd_round = (L.bm.Bm == 1 && L.bm.Hm == 1 && R % 8 == 0 && (R / 8) % a.G == 0) ? R : 0;
  const int grid = L.B * L.Hq * L.bm.NQB;
  if (grid == 0) return hipSuccess;
  if (L.D == 128) return dispatch_mask<128>(a, L.mask_kind, L.score_kind, grid, stream);
  return dispatch_mask<64>(a, L.mask_kind, L.score_kind, grid, stream);
}

}  // namespace fa
