// fa_fwd_split.hpp — merge of split-KV partial results (gfx950).
//
// A split-KV pass runs the FA2-order forward on disjoint key ranges of the same query
// rows; split s leaves, per row, its normalized partial output O_s and its partial
// logsumexp L_s. Merging is the online-softmax block merge of [P1] currybab.bearblog.dev
// ("Online Softmax 개념": the statistics of two blocks are combined by rescaling each to
// the larger maximum) and of the worked [1,2,3,4] split in [P3] ariser.io ("소프트맥스는 나누어
// 계산할 수 있다"), written in logsumexp form:
//     L = log sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s.
// A split whose keys are all masked for a row has L_s = -inf and weight 0.
#pragma once

#include "fa_common.hpp"

namespace fa {

// One row per 16 threads; each thread merges D / 16 columns. rows = B * H * N; the
// partial arrays are [n_split][rows][D] and [n_split][rows].
template <bool BF16, int D>
__global__ void __launch_bounds__(256) fa_split_merge_kernel(const float* __restrict__ o_part,
                                                             const float* __restrict__ l_part,
                                                             uint16_t* __restrict__ o,
                                                             float* __restrict__ lse,
                                                             long long rows, int n_split) {
  using E = Elt<BF16>;
  constexpr int TPR = 16, CPT = D / TPR;  // threads per row, columns per thread (4 or 8)
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= rows) return;
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.69314718055994530942f;
  float mx = -__builtin_inff();
  for (int s = 0; s < n_split; ++s) mx = __builtin_fmaxf(mx, l_part[s * rows + row]);
  float sum = 0.f;
  for (int s = 0; s < n_split; ++s)
    sum += __builtin_amdgcn_exp2f((l_part[s * rows + row] - mx) * kLog2e);
  const float L = mx + __builtin_amdgcn_logf(sum) * kLn2;
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float w = __builtin_amdgcn_exp2f((l_part[s * rows + row] - L) * kLog2e);
    const float* src = o_part + ((size_t)s * rows + row) * D + part * CPT;
#pragma unroll
    for (int c = 0; c < CPT; c += 4) {
      const float4 x = *reinterpret_cast<const float4*>(src + c);
      acc[c] += w * x.x;
      acc[c + 1] += w * x.y;
      acc[c + 2] += w * x.z;
      acc[c + 3] += w * x.w;
    }
  }
  uint16_t* dst = o + row * D + part * CPT;
#pragma unroll
  for (int c = 0; c < CPT; c += 4)
    *reinterpret_cast<u32x2_t*>(dst + c) =
        u32x2_t{E::pack(acc[c], acc[c + 1]), E::pack(acc[c + 2], acc[c + 3])};
  if (part == 0) lse[row] = L;
}

}  // namespace fa
