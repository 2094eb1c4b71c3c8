// fa_bwd.hip — host side of the backward entry points declared in include/fa.h:
// validation (entirely before any HIP call) and dispatch to the launches of the head dim.
#include "fa.h"
#include "fa_bwd.hpp"
#include "fa_host.hpp"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

// The launches live in fa_bwd_d64.hip and fa_bwd_d128.hip (one translation unit per
// head dim, each compiled with its own options); nothing here instantiates them.
namespace fa {
extern template hipError_t launch_bwd<true, 64, false>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd<true, 64, true>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd<false, 64, false>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd<false, 64, true>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd<true, 128, false>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd<true, 128, true>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd<false, 128, false>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd<false, 128, true>(const BwdParams&, hipStream_t);
}  // namespace fa

namespace {

using fa::kBwdRows;

int validate_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, const void* dq, const void* dk, const void* dv, int B, int H,
                 int N, int d, float scale) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(N) * d >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t bh = static_cast<int64_t>(B) * H;
  if (bh >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t rows = bh * N;
  if (rows > (int64_t(1) << 54)) return FA_ERR_SHAPE;
  const int64_t tiles = (N + kBwdRows - 1) / kBwdRows;
  if (tiles * bh >= (int64_t(1) << 31) / 64) return FA_ERR_SHAPE;  // grid limit
  const uint64_t tb = static_cast<uint64_t>(rows * d) * 2u;
  const uint64_t lb = static_cast<uint64_t>(rows) * 4u;
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                        reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if ((a16 & 15u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_ALIGN;
  // each output may overlap neither another output nor any input
  const void* outs[3] = {dq, dk, dv};
  const void* ins[6] = {q, k, v, o, dout, lse};
  const uint64_t in_bytes[6] = {tb, tb, tb, tb, tb, lb};
  for (int a = 0; a < 3; ++a) {
    for (int b = a + 1; b < 3; ++b)
      if (fa_host::ranges_overlap(outs[a], tb, outs[b], tb)) return FA_ERR_ALIAS;
    for (int b = 0; b < 6; ++b)
      if (fa_host::ranges_overlap(outs[a], tb, ins[b], in_bytes[b])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

template <bool BF16>
int fa_bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, void* stream) {
  const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale);
  if (st != FA_OK) return st;
  fa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.lse = lse;
  p.dout = static_cast<const uint16_t*>(dout);
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  // D and L log2(e): 2 B*H*N floats, within dq's B*H*N*d*2 bytes (d >= 64)
  p.delta = static_cast<float*>(dq);
  p.lse2 = p.delta + static_cast<size_t>(B) * H * N;
  p.N = N;
  p.BH = B * H;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  hipError_t e;
  if (d == 128)
    e = cz ? fa::launch_bwd<BF16, 128, true>(p, s) : fa::launch_bwd<BF16, 128, false>(p, s);
  else e = cz ? fa::launch_bwd<BF16, 64, true>(p, s) : fa::launch_bwd<BF16, 64, false>(p, s);
  if (e != hipSuccess) {
    fa_host::g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, void* stream) {
  return fa_bwd_impl<true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, stream);
}

int fa_bwd_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, void* stream) {
  return fa_bwd_impl<false>(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal,
                            stream);
}

}  // extern "C"
