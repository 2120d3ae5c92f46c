// Block-sparse attention forward with fp16 inputs: the kernel of
// fwd_bf16_kernel.hpp with the fp16 element type (fp16 MFMA, P rounded to
// fp16), contiguous K/V, with split-KV (page "tensorplay.nn.attention API",
// whose worked example runs the forward on fp16 tensors).
#include "fwd_bf16_kernel.hpp"

namespace fa {

hipError_t launch_fwd_f16(const FwdLaunch& L, hipStream_t stream) {
  return launch_impl<false, true>(L, stream);
}

}  // namespace fa
