// fa_bwd_d128.hip — the backward kernels and launches at head dim 128 (bfloat16 and
// float16, with and without the causal mask), one translation unit per head dim so that
// each is compiled with its own code-generation options.
//
// Compiled with LLVM's iterative ILP machine scheduler (see build.py) for the 32-key
// dK/dV kernel of fa_bwd.hpp (taken at a zero scale): it runs one wave per SIMD with more
// than 256 registers, and the default scheduler issues each product's LDS operand read
// just before the product; the ILP schedule issues the reads earlier. The kernels of
// fa_bwd_wide.hpp fix their own order with scheduling barriers.
#include "fa_bwd_wide.hpp"

namespace fa {
template hipError_t launch_bwd<true, 128, false>(const BwdParams&, hipStream_t);
template hipError_t launch_bwd<true, 128, true>(const BwdParams&, hipStream_t);
template hipError_t launch_bwd<false, 128, false>(const BwdParams&, hipStream_t);
template hipError_t launch_bwd<false, 128, true>(const BwdParams&, hipStream_t);
}  // namespace fa
