// fa_bwd_d64.hip — the backward kernels and launches at head dim 64 (bfloat16 and
// float16, with and without the causal mask), one translation unit per head dim so that
// each is compiled with its own code-generation options.
#include "fa_bwd_wide.hpp"

namespace fa {
template hipError_t launch_bwd<true, 64, false>(const BwdParams&, hipStream_t);
template hipError_t launch_bwd<true, 64, true>(const BwdParams&, hipStream_t);
template hipError_t launch_bwd<false, 64, false>(const BwdParams&, hipStream_t);
template hipError_t launch_bwd<false, 64, true>(const BwdParams&, hipStream_t);
}  // namespace fa
