// Block-sparse attention forward, bf16, contiguous K/V (the kernel and its
// design notes are in fwd_bf16_kernel.hpp); paged K/V dispatch to
// fwd_bf16_paged.hip, a separate translation unit so both compile in
// parallel.
#include "fwd_bf16_kernel.hpp"

namespace fa {

int fwd_bf16_lds_bytes(int D, int NKB, bool paged) {
  (void)D;
  return 4 * kStepBytes + 4 * ((NKB + 3) & ~3) * (paged ? 2 : 1) + 2 * 128 * 4;
}

hipError_t launch_fwd_bf16(const FwdLaunch& L, hipStream_t stream) {
  if (L.f16) return launch_fwd_f16(L, stream);
  if (L.page_table) return launch_fwd_bf16_paged(L, stream);
  return launch_impl<false, false>(L, stream);
}

}  // namespace fa
