// Block-sparse attention forward, bf16, over a paged KV cache: the kernel of
// fwd_bf16_kernel.hpp with per-tile page translation (page "FlagAttention",
// operator overview: paged attention over a KV cache kept in pages).
#include "fwd_bf16_kernel.hpp"

namespace fa {

hipError_t launch_fwd_bf16_paged(const FwdLaunch& L, hipStream_t stream) {
  return launch_impl<true, false>(L, stream);
}

}  // namespace fa
