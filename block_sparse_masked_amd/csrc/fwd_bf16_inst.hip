// Explicit instantiations of one slice of the 16-bit forward kernels (every
// mask kind x score kind x MFMA step for one head dim, KV layout and element
// type). The build compiles this file once per slice with FA_D (64, 128 or
// 256), FA_PAGED (0 or 1) and FA_F16 (0 or 1) defined, so the slices compile
// in parallel; fwd_bf16.hip declares them all and dispatches at run time.
#include "fwd_bf16_kernel.hpp"

#if !defined(FA_D) || !defined(FA_PAGED) || !defined(FA_F16)
#error "compile fwd_bf16_inst.hip with -DFA_D=<64|128|256> -DFA_PAGED=<0|1> -DFA_F16=<0|1>"
#endif

namespace fa {

FA_FWD16_SLICE(FA_D, FA_PAGED != 0, FA_F16 != 0);

}  // namespace fa
