// Launcher of the 16-bit block-sparse attention forward (the kernel and its
// design notes are in fwd_bf16_kernel.hpp): argument set-up, the launch plan
// (fwd_plan.hpp), dispatch to the kernel instantiations of
// fwd_bf16_inst.hip, and the merge of split-KV slices.
#include <mutex>

#include "fwd_bf16_kernel.hpp"

namespace fa {

// the instantiations live in fwd_bf16_inst.hip's objects
FA_FWD16_SLICES(extern);

namespace {

// Merge of the split-KV slices, one 64-lane wave per query row: with the
// slices' LSE_s, LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s
// (the rescaling of the online softmax, applied across slices).
template <int D, bool F16>
__global__ __launch_bounds__(256) void splitkv_combine_kernel(FwdArgs a) {
  using T = typename Elem<F16>::T;
  constexpr int PER = D / 64;  // elements per lane
  const long long rows = (long long)a.B * a.Hq * a.Q_LEN;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  // slices are read in batches of 8 (indices clamped to the last slice, the
  // extra ones weighted 0) so the batch's loads are in flight together
  constexpr int BATCH = 8;
  float m = -INFINITY;
  for (int s0 = 0; s0 < a.splits; s0 += BATCH) {
    float ls[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) ls[u] = a.part_lse[min(s0 + u, a.splits - 1) * rows + row];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) m = fmaxf(m, ls[u]);
  }
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float wsum = 0.0f;
  if (m != -INFINITY) {
    for (int s0 = 0; s0 < a.splits; s0 += BATCH) {
      float ls[BATCH], ov[BATCH][PER];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const long long srow = (long long)min(s0 + u, a.splits - 1) * rows + row;
        ls[u] = a.part_lse[srow];
        __builtin_memcpy(ov[u], a.part_o + srow * D + lane * PER, PER * 4);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const float w = (s0 + u >= a.splits || ls[u] == -INFINITY)
                            ? 0.0f : fast_exp2((ls[u] - m) * kLog2e);
        wsum += w;
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, ov[u][i], acc[i]);
      }
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  const int qi = (int)(row % a.Q_LEN);
  const long long bh = row / a.Q_LEN;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  u16* orow = a.o + b * a.so0 + h * a.so1 + (long long)qi * a.so2 + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const T v = (T)(acc[i] * inv);
    __builtin_memcpy(orow + i, &v, 2);
  }
  if (lane == 0)
    a.lse[((long long)b * a.Hq + h) * a.Q_LEN + qi] =
        wsum > 0.0f ? m + fast_log2(wsum) * kLn2 : -INFINITY;
}


// Argument set-up, launch shape and dispatch of the forward (and the merge
// of split-KV slices); PAGED selects the paged-KV instantiations.
template <bool PAGED, bool F16>
hipError_t launch_impl(const FwdLaunch& L, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const u16*>(L.q);
  a.k = static_cast<const u16*>(L.k);
  a.v = static_cast<const u16*>(L.v);
  a.o = static_cast<u16*>(L.o);
  a.lse = L.lse;
  a.sq0 = L.sq[0]; a.sq1 = L.sq[1]; a.sq2 = L.sq[2];
  a.sk0 = L.sk[0]; a.sk1 = L.sk[1]; a.sk2 = (int)L.sk[2];
  a.sv0 = L.sv[0]; a.sv1 = L.sv[1]; a.sv2 = (int)L.sv[2];
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
  a.splits = L.splits > 1 ? L.splits : 1;
  a.part_o = L.part_o;
  a.part_lse = L.part_lse;
  a.page_table = L.page_table;
  a.page_size = L.page_size;
  a.pt_stride = L.pt_stride;
  a.num_pages = L.num_pages;
  a.o32 = L.o32;
  // query heads per workgroup, MFMA step and the XCD remap (the rule is
  // shared with flexattn_fwd_make_plan)
  const FwdPlan plan = plan_fwd(L.B, L.Hq, L.Hkv, L.Q_LEN, L.D, L.bm.Bm, L.bm.Hm, L.bm.NQB,
                                L.bm.QBS, L.bm.NKB, 0);
  a.wph = plan.wph;
  a.xcd_round = plan.xcd_round;
  const long long grid_ll = plan.items * a.splits;
  if (grid_ll > 0x7fffffffLL) return hipErrorInvalidValue;
  const int grid = (int)grid_ll;
  if (grid == 0) return hipSuccess;
  // the unscaled fast path takes the row max before scaling: scale must be > 0
  const int score = (L.score_kind == SCORE_NONE && !(L.scale > 0.0f)) ? SCORE_SCALED : L.score_kind;
  hipError_t e = (L.D == 256) ? fwd16_launch<256, PAGED, F16>(a, plan.r16, L.mask_kind, score, grid, stream)
               : (L.D == 128) ? fwd16_launch<128, PAGED, F16>(a, plan.r16, L.mask_kind, score, grid, stream)
                              : fwd16_launch<64, PAGED, F16>(a, plan.r16, L.mask_kind, score, grid, stream);
  if (e != hipSuccess || a.splits == 1) return e;
  const long long rows = (long long)L.B * L.Hq * L.Q_LEN;
  const unsigned blocks = (unsigned)((rows + 3) / 4);
  if (L.D == 256) splitkv_combine_kernel<256, F16><<<blocks, 256, 0, stream>>>(a);
  else if (L.D == 128) splitkv_combine_kernel<128, F16><<<blocks, 256, 0, stream>>>(a);
  else splitkv_combine_kernel<64, F16><<<blocks, 256, 0, stream>>>(a);
  return hipGetLastError();
}


}  // namespace

// Scratch of the allocation-free split-KV entry point: the slices' fp32
// partial O and LSE. One copy per GPU, held until the process ends; every
// call on a GPU reuses it (calls that overlap on one GPU race).
__device__ __align__(256) float scratch[kFwdScratchBytes / sizeof(float)];

hipError_t fwd_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // the array's device address on this GPU (its name is a host-side
    // stand-in that must never reach a kernel)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kFwdScratchBytes;
  return hipSuccess;
}

int fwd_bf16_lds_bytes(int D, int NKB, bool paged) {
  const int step = D == 64 ? step_bytes<64>() : kStepBytes;
  return 4 * step + 4 * ((NKB + 3) & ~3) * (paged ? 2 : 1) + 2 * 128 * 4;
}

hipError_t launch_fwd_bf16(const FwdLaunch& L, hipStream_t stream) {
  if (L.f16) return L.page_table ? launch_impl<true, true>(L, stream)
                                  : launch_impl<false, true>(L, stream);
  if (L.page_table) return launch_impl<true, false>(L, stream);
  return launch_impl<false, false>(L, stream);
}

}  // namespace fa
