// Block-sparse attention forward, fp32 inputs, fp32 arithmetic throughout
// (no bf16 or reduced-precision matrix path), gfx950.
//
// Same method as the bf16 forward (page "tensorplay.nn.attention API",
// BlockMask "Details" items 1-2: per-row tile lists, mask_mod only on partial
// tiles; online softmax over KV tiles), with plain fp32 FMA on the vector
// ALUs, in natural-log units with accurate tanh / exp / log. One workgroup
// of 128 threads per 32 query rows of a (b, h, 128-row query tile) -- four
// workgroups per tile, so small problems still spread over many CUs; each
// query row is shared by four threads that split the head dimension.
#include "common.hpp"
#include "fwd_common.hpp"
#include "launch.hpp"

namespace fa {

namespace {

constexpr int kTpr = 4;                        // threads per query row
constexpr int kRowsPerWg = 32;                 // query rows per workgroup
constexpr int kThreads = kTpr * kRowsPerWg;
constexpr int kChunk = 16;  // keys per online-softmax update
constexpr int kSub = 64;    // keys staged in LDS at a time (half a tile)

// score_mod in natural units with the accurate libm-style device functions:
// scale * s, then softcap * tanh(. / softcap), then + m_h * (kv - q).
template <int SCORE>
__device__ __forceinline__ float score_natural(float s, float scale, float cap, float slope,
                                               float dist) {
  float t = s * scale;
  if constexpr (SCORE == SCORE_SOFTCAP || SCORE == SCORE_SOFTCAP_ALIBI) t = cap * tanhf(t / cap);
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI) t = fmaf(slope, dist, t);
  return t;
}

// Sum over the four lanes of a quad (the threads of one query row), with DPP
// quad permutations: xor 1, then xor 2.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  return x;
}

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  long long sq0, sq1, sq2, sk0, sk1, sk2, sv0, sv1, sv2, so0, so1, so2;
  int B, Hq, G, Q_LEN, KV_LEN;
  MaskParams mp;
  float scale, softcap;
  const float* slopes;
  BlockMaskView bm;
};

template <int D>
__device__ __forceinline__ void load_tile_f32(float* lds, const float* g, long long row_stride,
                                              int kv0, int kv_len) {
  constexpr int CPR = D / 4;  // float4 chunks per row
  constexpr int N = kSub * CPR / kThreads;
#pragma unroll 8
  for (int i = 0; i < N; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c / CPR;
    const int col = c % CPR;
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    if (kv0 + row < kv_len)
      val = *reinterpret_cast<const float4*>(g + (long long)(kv0 + row) * row_stride + col * 4);
    *reinterpret_cast<float4*>(lds + row * D + col * 4) = val;
  }
}

template <int D, int MASK, int SCORE>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args a) {
  constexpr int HD = D / kTpr;  // dims per thread
  extern __shared__ float smem_f32[];
  float* sK = smem_f32;
  float* sV = smem_f32 + kSub * D;

  // kRowsPerWg query rows per workgroup, BLOCK_SIZE / kRowsPerWg per tile row
  const int wg_per_row = a.bm.QBS / kRowsPerWg;
  const Item it = decode_item(blockIdx.x / wg_per_row, a.bm, a.B, a.Hq);
  const int b = it.b, h = it.h, hk = h / a.G;
  const int half = threadIdx.x % kTpr;  // this thread's quarter of the head dimension
  const int q = it.qb * a.bm.QBS + (blockIdx.x % wg_per_row) * kRowsPerWg + threadIdx.x / kTpr;
  const bool qvalid = q < a.Q_LEN;
  const int qc = qvalid ? q : a.Q_LEN - 1;

  float qv[HD];
  {
    const float* qrow = a.q + b * a.sq0 + h * a.sq1 + (long long)qc * a.sq2 + half * HD;
#pragma unroll
    for (int d = 0; d < HD; d += 4) {
      const float4 t4 = *reinterpret_cast<const float4*>(qrow + d);
      qv[d] = t4.x; qv[d + 1] = t4.y; qv[d + 2] = t4.z; qv[d + 3] = t4.w;
    }
  }
  float acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) acc[d] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  float slope = 0.0f;
  if constexpr (SCORE == SCORE_ALIBI || SCORE == SCORE_SOFTCAP_ALIBI)
    slope = alibi_slope(a.slopes, h, a.Hq);
  const int* doc = (mask_uses_doc(MASK) && a.mp.doc) ? a.mp.doc + b * a.mp.doc_bstride : nullptr;

  const float* kbase = a.k + b * a.sk0 + hk * a.sk1;
  const float* vbase = a.v + b * a.sv0 + hk * a.sv1;
  const long long lrow = (long long)it.mrow * a.bm.NKB;
  const int nfull = a.bm.full_num[it.mrow];
  const int npart = a.bm.kv_num[it.mrow];

  for (int t = 0; t < nfull + npart; ++t) {
    const bool partial = t >= nfull;
    const int kb = partial ? a.bm.kv_idx[lrow + (t - nfull)] : a.bm.full_idx[lrow + t];
    const bool do_mask = partial || (kb * a.bm.BS + a.bm.BS > a.KV_LEN);
   for (int sub = 0; sub < a.bm.BS; sub += kSub) {
    const int kv0 = kb * a.bm.BS + sub;
    __syncthreads();
    load_tile_f32<D>(sK, kbase, a.sk2, kv0, a.KV_LEN);
    load_tile_f32<D>(sV, vbase, a.sv2, kv0, a.KV_LEN);
    __syncthreads();

    for (int c0 = 0; c0 < kSub; c0 += kChunk) {
      float x[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const float4* krow = reinterpret_cast<const float4*>(sK + (c0 + j) * D + half * HD);
        float part = 0.0f;
#pragma unroll
        for (int d4 = 0; d4 < HD / 4; ++d4) {
          const float4 kk = krow[d4];
          part = fmaf(qv[4 * d4], kk.x, part);
          part = fmaf(qv[4 * d4 + 1], kk.y, part);
          part = fmaf(qv[4 * d4 + 2], kk.z, part);
          part = fmaf(qv[4 * d4 + 3], kk.w, part);
        }
        const float sdot = quad_sum(part);
        const int key = kv0 + c0 + j;
        float xv = score_natural<SCORE>(sdot, a.scale, a.softcap, slope, (float)(key - q));
        if (do_mask) {
          const bool ok =
              key < a.KV_LEN && (partial ? Mask<MASK>::allowed(a.mp, doc, qc, key) : true);
          xv = ok ? xv : -INFINITY;
        }
        x[j] = xv;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) mx = fmaxf(mx, x[j]);
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = expf(m - m_use);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc[d] *= alpha;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const float p = expf(x[j] - m_use);
        l += p;
        const float4* vrow = reinterpret_cast<const float4*>(sV + (c0 + j) * D + half * HD);
#pragma unroll
        for (int d4 = 0; d4 < HD / 4; ++d4) {
          const float4 vv = vrow[d4];
          acc[4 * d4] = fmaf(p, vv.x, acc[4 * d4]);
          acc[4 * d4 + 1] = fmaf(p, vv.y, acc[4 * d4 + 1]);
          acc[4 * d4 + 2] = fmaf(p, vv.z, acc[4 * d4 + 2]);
          acc[4 * d4 + 3] = fmaf(p, vv.w, acc[4 * d4 + 3]);
        }
      }
      m = m_new;
    }
   }
  }

  if (qvalid) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* orow = a.o + b * a.so0 + h * a.so1 + (long long)q * a.so2 + half * HD;
#pragma unroll
    for (int d = 0; d < HD; d += 4) {
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
    }
    if (half == 0) {
      const float lse = l > 0.0f ? m + logf(l) : -INFINITY;
      a.lse[((long long)b * a.Hq + h) * a.Q_LEN + q] = lse;
    }
  }
}

template <int D, int MASK>
hipError_t f32_dispatch_score(const F32Args& args, int score, int grid, hipStream_t stream) {
  const size_t lds = sizeof(float) * 2 * kSub * D;
  switch (score) {
    case SCORE_NONE:
      fwd_f32_kernel<D, MASK, SCORE_NONE><<<grid, kThreads, lds, stream>>>(args);
      break;
    case SCORE_ALIBI:
      fwd_f32_kernel<D, MASK, SCORE_ALIBI><<<grid, kThreads, lds, stream>>>(args);
      break;
    case SCORE_SOFTCAP:
      fwd_f32_kernel<D, MASK, SCORE_SOFTCAP><<<grid, kThreads, lds, stream>>>(args);
      break;
    default:
      fwd_f32_kernel<D, MASK, SCORE_SOFTCAP_ALIBI><<<grid, kThreads, lds, stream>>>(args);
      break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t f32_dispatch_mask(const F32Args& args, int mask, int score, int grid,
                             hipStream_t stream) {
  switch (mask) {
    case MASK_NOOP:
      return f32_dispatch_score<D, MASK_NOOP>(args, score, grid, stream);
    case MASK_CAUSAL:
      return f32_dispatch_score<D, MASK_CAUSAL>(args, score, grid, stream);
    case MASK_SLIDING_SINK:
      return f32_dispatch_score<D, MASK_SLIDING_SINK>(args, score, grid, stream);
    case MASK_PREFIX_LM:
      return f32_dispatch_score<D, MASK_PREFIX_LM>(args, score, grid, stream);
    case MASK_COMPOSITE:
      return f32_dispatch_score<D, MASK_COMPOSITE>(args, score, grid, stream);
    default:
      return f32_dispatch_score<D, MASK_DOCUMENT>(args, score, grid, stream);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdLaunch& L, hipStream_t stream) {
  F32Args a;
  a.q = static_cast<const float*>(L.q);
  a.k = static_cast<const float*>(L.k);
  a.v = static_cast<const float*>(L.v);
  a.o = static_cast<float*>(L.o);
  a.lse = L.lse;
  a.sq0 = L.sq[0]; a.sq1 = L.sq[1]; a.sq2 = L.sq[2];
  a.sk0 = L.sk[0]; a.sk1 = L.sk[1]; a.sk2 = L.sk[2];
  a.sv0 = L.sv[0]; a.sv1 = L.sv[1]; a.sv2 = L.sv[2];
  a.so0 = L.so[0]; a.so1 = L.so[1]; a.so2 = L.so[2];
  a.B = L.B;
  a.Hq = L.Hq;
  a.G = L.Hq / L.Hkv;
  a.Q_LEN = L.Q_LEN;
  a.KV_LEN = L.KV_LEN;
  a.mp = L.mp;
  a.scale = L.scale;
  a.softcap = L.softcap;
  a.slopes = L.slopes;
  a.bm = L.bm;
  const int grid = L.B * L.Hq * L.bm.NQB * (L.bm.QBS / kRowsPerWg);
  if (grid == 0) return hipSuccess;
  if (L.D == 128) return f32_dispatch_mask<128>(a, L.mask_kind, L.score_kind, grid, stream);
  return f32_dispatch_mask<64>(a, L.mask_kind, L.score_kind, grid, stream);
}

}  // namespace fa
