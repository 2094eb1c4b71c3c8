// fa_fwd.hip — host side of the C ABI declared in include/fa.h: argument
// validation (entirely before any HIP call), kernel selection and launch.
#include "fa.h"
#include "fa_fwd_kernel.hpp"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kNW = 4;   // waves per workgroup
constexpr int kQB = 1;   // 32-query blocks per wave
constexpr int kBC = 64;  // keys per tile

bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int B, int H, int N, int d, float scale) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SHAPE;
  if (d > 128) return FA_ERR_UNSUPPORTED;
  // N*d indexes one head with 32-bit row arithmetic; B*H*N*d*2 bytes must be addressable
  if (static_cast<int64_t>(N) * d >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t bh = static_cast<int64_t>(B) * H;
  if (bh >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t rows = bh * N;                       // < 2^62
  if (rows > (int64_t(1) << 54)) return FA_ERR_SHAPE;
  const int64_t elems = rows * d;                    // < 2^61
  const int64_t n_qt = (N + kNW * kQB * 32 - 1) / (kNW * kQB * 32);
  if (n_qt * bh >= (int64_t(1) << 31) / 64) return FA_ERR_SHAPE;   // grid limit
  const uint64_t tbytes = static_cast<uint64_t>(elems) * 2u;
  const uint64_t lbytes = static_cast<uint64_t>(rows) * 4u;
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if ((a16 & 15u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_ALIGN;
  if (ranges_overlap(o, tbytes, q, tbytes) || ranges_overlap(o, tbytes, k, tbytes) ||
      ranges_overlap(o, tbytes, v, tbytes) || ranges_overlap(lse, lbytes, q, tbytes) ||
      ranges_overlap(lse, lbytes, k, tbytes) || ranges_overlap(lse, lbytes, v, tbytes) ||
      ranges_overlap(lse, lbytes, o, tbytes))
    return FA_ERR_ALIAS;
  return FA_OK;
}

template <bool BF16, int D, bool EXACT_D, bool CAUSAL>
hipError_t launch_one(const fa::Params& p, int grid, hipStream_t stream) {
  auto kern = fa::fa_fwd_kernel<BF16, D, EXACT_D, CAUSAL, kQB, kNW, kBC>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kNW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16>
int fa_fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int N, int d, float scale, int causal, void* stream) {
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale);
  if (st != FA_OK) return st;

  constexpr int BR = kNW * kQB * 32;
  fa::Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.N = N;
  p.d = d;
  p.BH = B * H;
  p.n_qt = (N + BR - 1) / BR;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  p.qsign = std::signbit(scale) ? 0x80008000u : 0u;
  p.xcd_map = (p.BH % 8) == 0 ? 1 : 0;
  const int grid = p.n_qt * p.BH;
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e;
  const bool cz = causal != 0;
  if (d <= 64) {
    if (d == 64) e = cz ? launch_one<BF16, 64, true, true>(p, grid, s)
                        : launch_one<BF16, 64, true, false>(p, grid, s);
    else e = cz ? launch_one<BF16, 64, false, true>(p, grid, s)
                : launch_one<BF16, 64, false, false>(p, grid, s);
  } else {
    if (d == 128) e = cz ? launch_one<BF16, 128, true, true>(p, grid, s)
                         : launch_one<BF16, 128, true, false>(p, grid, s);
    else e = cz ? launch_one<BF16, 128, false, true>(p, grid, s)
                : launch_one<BF16, 128, false, false>(p, grid, s);
  }
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, void* stream) {
  return fa_fwd_impl<true>(q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int N, int d, float scale, int causal, void* stream) {
  return fa_fwd_impl<false>(q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_supported(int d, int dtype, int causal) {
  (void)causal;
  if (d < 1 || d > 128) return 0;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return 0;
  return 1;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape or scale (B, H, N, d >= 1; finite scale; sizes in range)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (1 <= d <= 128) or dtype";
    case FA_ERR_ALIAS: return "o or lse overlaps q, k, v or each other";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_HIP: return "the HIP runtime refused the launch (see fa_last_hip_error)";
    default: return "unknown status";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

const char* fa_version(void) { return "fa355 0.1.0 (gfx950, FA2 forward)"; }

}  // extern "C"
