// Matrix-core throughput probe (measurement aid, not part of the attention
// path): every wave issues v_mfma_f32_32x32x16_bf16 back to back on four
// independent accumulators, so the chip's sustained dense bf16 MFMA rate at
// the clock it actually runs under a full matrix load can be timed beside the
// published peak (256 CUs x 4096 flop/clk x 2.4 GHz). Built into its own
// library, libfaprobe.so, which only the benchmark loads.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(lane + i));
    b[i] = (__bf16)(1e-3f * (float)(lane - i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Runs `blocks` workgroups of 4 waves, each wave issuing 4 * iters MFMAs of
// 32 x 32 x 16 (32768 flops each), on `stream`. out: device float[blocks * 256]
// (each lane's accumulator sum, written so the work is not optimised away).
// Returns 0, or the HIP error of the launch.
extern "C" int faprobe_mfma_bf16(int iters, int blocks, float* out, hipStream_t stream) {
  if (iters <= 0 || blocks <= 0 || out == nullptr) return (int)hipErrorInvalidValue;
  mfma_probe_kernel<<<blocks, 256, 0, stream>>>(iters, out);
  return (int)hipGetLastError();
}
