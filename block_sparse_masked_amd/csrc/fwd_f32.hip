// Block-sparse attention forward, fp32 inputs, fp32 arithmetic throughout
// (no bf16 or reduced-precision matrix path), gfx950.
//
// Same method as the bf16 forward (page "tensorplay.nn.attention API",
// BlockMask "Details" items 1-2: per-row tile lists, mask_mod only on partial
// tiles; online softmax over KV tiles), with plain fp32 FMA on the vector
// ALUs, in natural-log units with accurate tanh / exp / log.
//
// One workgroup of 256 threads per 8 query rows of a (b, h, query tile), so
// small problems still spread over many CUs. Each row has 32 threads: eight
// key groups of four threads, the four splitting the head dimension. Key
// group g takes the keys g, g + 8, g + 16, ... of every block of keys staged
// in LDS and keeps its own online softmax (max, sum, output) over them, so a
// thread's serial chain covers an eighth of the row's keys and every
// exponential is computed once per key group rather than once per row
// thread. The next block's K and V are loaded into registers while a block
// is computed. At the end the groups' partial results are merged through
// LDS with the softmax's own rescaling.
#include "common.hpp"
#include "fwd_common.hpp"
#include "launch.hpp"

namespace fa {

namespace {

constexpr int kTpr = 4;         // threads per (row, key group): head-dim quarters
constexpr int kGroups = 8;      // key groups per row
constexpr int kRowsPerWg = kF32RowsPerWorkgroup;  // query rows per workgroup
constexpr int kThreads = kTpr * kGroups * kRowsPerWg;

// keys staged in LDS at a time, and the LDS row stride (floats): 4 floats of
// padding put consecutive keys, which neighbouring key groups read at once,
// on different banks
template <int D>
struct F32Geom {
  static constexpr int SUB = D >= 128 ? 32 : 64;
  static constexpr int PER = SUB / kGroups;  // keys of a group per staged block
  static constexpr int LD = D + 4;
  static constexpr int HD = D / kTpr;        // head dims per thread
  static constexpr int STAGE = 2 * SUB * LD;
  static constexpr int MERGE = kThreads * (2 + HD);
  static constexpr size_t LDS = sizeof(float) * (STAGE > MERGE ? STAGE : MERGE);
};

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

// Sum over the four lanes of a quad (the threads of one row's key group),
// with DPP quad permutations: xor 1, then xor 2.
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

// Staging of keys [kv0, kv0 + SUB) of a [len][D] matrix: each thread loads
// its N float4 chunks into registers (rows at or past kv_len read as zero),
// and later stores them to LDS rows of LD floats, so the loads of the next
// block are in flight while the current one is computed.
template <int D>
struct StageF32 {
  using F = F32Geom<D>;
  static constexpr int CPR = D / 4;  // float4 chunks per row
  static constexpr int N = F::SUB * CPR / kThreads;
  float4 r[N];
  __device__ __forceinline__ void load(const float* g, long long row_stride, int kv0,
                                       int kv_len) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int row = c / CPR;
      r[i] = kv0 + row < kv_len
                 ? *reinterpret_cast<const float4*>(g + (long long)(kv0 + row) * row_stride +
                                                    (c % CPR) * 4)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __device__ __forceinline__ void store(float* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + kThreads * i;
      *reinterpret_cast<float4*>(lds + (c / CPR) * F::LD + (c % CPR) * 4) = r[i];
    }
  }
};

template <int D, int MASK, int SCORE>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(F32Args a) {
  using F = F32Geom<D>;
  constexpr int HD = F::HD;
  constexpr int PER = F::PER;
  extern __shared__ float smem_f32[];
  float* sK = smem_f32;
  float* sV = smem_f32 + F::SUB * F::LD;

  // kRowsPerWg query rows per workgroup, BLOCK_SIZE / kRowsPerWg per tile row
  const int wg_per_row = a.bm.QBS / kRowsPerWg;
  const Item it = decode_item(blockIdx.x / wg_per_row, a.bm, a.B, a.Hq);
  const int b = it.b, h = it.h, hk = h / a.G;
  const int dq = threadIdx.x % kTpr;              // this thread's quarter of the head dimension
  const int kg = (threadIdx.x / kTpr) % kGroups;  // its key group
  const int rl = threadIdx.x / (kTpr * kGroups);  // its row within the workgroup
  const int q = it.qb * a.bm.QBS + (blockIdx.x % wg_per_row) * kRowsPerWg + rl;
  const bool qvalid = q < a.Q_LEN;
  const int qc = qvalid ? q : a.Q_LEN - 1;

  float qv[HD];
  {
    const float* qrow = a.q + b * a.sq0 + h * a.sq1 + (long long)qc * a.sq2 + dq * HD;
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

  // the row's keys in blocks of SUB: block s is part s % spt of listed tile
  // s / spt (full tiles first); the next block's K and V are loaded into
  // registers while block s is computed
  const int spt = a.bm.BS / F::SUB;
  const int nblk = (nfull + npart) * spt;
  auto block_kv0 = [&](int s) {
    const int t = s / spt;
    const int kb = t >= nfull ? a.bm.kv_idx[lrow + (t - nfull)] : a.bm.full_idx[lrow + t];
    return kb * a.bm.BS + (s - t * spt) * F::SUB;
  };
  StageF32<D> stk, stv;
  if (nblk > 0) {
    const int kv0 = block_kv0(0);
    stk.load(kbase, a.sk2, kv0, a.KV_LEN);
    stv.load(vbase, a.sv2, kv0, a.KV_LEN);
  }
  for (int s = 0; s < nblk; ++s) {
    const int t = s / spt;
    const bool partial = t >= nfull;
    const int kv0 = block_kv0(s);
    const bool do_mask = partial || (kv0 - (s - t * spt) * F::SUB + a.bm.BS > a.KV_LEN);
    __syncthreads();  // the previous block's LDS reads are done
    stk.store(sK);
    stv.store(sV);
    __syncthreads();
    if (s + 1 < nblk) {
      const int kv1 = block_kv0(s + 1);
      stk.load(kbase, a.sk2, kv1, a.KV_LEN);
      stv.load(vbase, a.sv2, kv1, a.KV_LEN);
    }

    // this key group's keys of the block: kg, kg + kGroups, ...
    float x[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int r = kGroups * j + kg;
      const float4* krow = reinterpret_cast<const float4*>(sK + r * F::LD + dq * HD);
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
      const int key = kv0 + r;
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
    for (int j = 0; j < PER; ++j) mx = fmaxf(mx, x[j]);
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = expf(m - m_use);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < HD; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const float p = expf(x[j] - m_use);
      l += p;
      const float4* vrow =
          reinterpret_cast<const float4*>(sV + (kGroups * j + kg) * F::LD + dq * HD);
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

  // merge the key groups: LSE = m + ln sum_g l_g e^{m_g - m},
  // O = sum_g acc_g e^{m_g - m} / that sum
  __syncthreads();  // the last block's LDS reads are done
  float* part = smem_f32 + threadIdx.x * (2 + HD);
  part[0] = m;
  part[1] = l;
#pragma unroll
  for (int d = 0; d < HD; ++d) part[2 + d] = acc[d];
  __syncthreads();
  if (kg != 0 || !qvalid) return;
  float mg[kGroups];
  float mt = -INFINITY;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    mg[g] = smem_f32[(threadIdx.x + g * kTpr) * (2 + HD)];
    mt = fmaxf(mt, mg[g]);
  }
  const float mt_use = (mt == -INFINITY) ? 0.0f : mt;
  float lt = 0.0f;
  float out[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) out[d] = 0.0f;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const float* pg = smem_f32 + (threadIdx.x + g * kTpr) * (2 + HD);
    const float w = expf(mg[g] - mt_use);  // 0 for a group with no allowed key
    lt = fmaf(pg[1], w, lt);
#pragma unroll
    for (int d = 0; d < HD; ++d) out[d] = fmaf(pg[2 + d], w, out[d]);
  }
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  float* orow = a.o + b * a.so0 + h * a.so1 + (long long)q * a.so2 + dq * HD;
#pragma unroll
  for (int d = 0; d < HD; d += 4) {
    *reinterpret_cast<float4*>(orow + d) =
        make_float4(out[d] * inv, out[d + 1] * inv, out[d + 2] * inv, out[d + 3] * inv);
  }
  if (dq == 0) {
    const float lse = lt > 0.0f ? mt + logf(lt) : -INFINITY;
    a.lse[((long long)b * a.Hq + h) * a.Q_LEN + q] = lse;
  }
}

template <int D, int MASK>
hipError_t f32_dispatch_score(const F32Args& args, int score, int grid, hipStream_t stream) {
  const size_t lds = F32Geom<D>::LDS;
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
