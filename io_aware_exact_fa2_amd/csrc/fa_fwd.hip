// fa_fwd.hip — host side of the C ABI declared in include/fa.h: argument
// validation (entirely before any HIP call), kernel selection and launch.
#include "fa.h"
#include "fa_fwd_fa1.hpp"
#include "fa_fwd_fast.hpp"
#include "fa_fwd_fp8.hpp"
#include "fa_fwd_split.hpp"
#include "fa_fwd_generic.hpp"
#include "fa_fwd_wide.hpp"
#include "fa_host.hpp"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

namespace {

using fa_host::cu_count;
using fa_host::g_last_hip_error;
using fa_host::ranges_overlap;

// Launch shapes. The fast paths (the 32-query kernel at d = 64, the wide kernel at
// d = 128) are tunable at build time for sweeps; the defaults are the measured best. The
// generic path (other d) is fixed.
#ifndef FA_FAST_NW
#define FA_FAST_NW 4      // waves per workgroup (8: -3% on the d = 64 workloads)
#endif
#ifndef FA_BC_D64
#define FA_BC_D64 64      // keys per tile at d = 64
#endif
#ifndef FA_WPE_D64
#define FA_WPE_D64 2      // least waves per SIMD the d = 64 kernel's registers must allow
#endif
#ifndef FA_QB_D64
#define FA_QB_D64 1       // 32-query blocks per wave at d = 64 (2: over 32-key tiles)
#endif
#ifndef FA_WIDE_RING
#define FA_WIDE_RING 4    // LDS ring slots per tensor
#endif
#ifndef FA_WIDE_BC
#define FA_WIDE_BC 64
#endif
constexpr int kFNW = FA_FAST_NW;
constexpr int kNW = 4;                    // generic path: waves per workgroup
constexpr int kQB = 1;                    //               32-query blocks per wave
constexpr int kBC = 64;                   //               keys per tile
constexpr int kGBR = kNW * kQB * 32;      //               queries per workgroup
constexpr int kMinBR = kFNW * 32 < kGBR ? kFNW * 32 : kGBR;   // smallest query tile

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int B, int H, int N, int d, float scale, float tau) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_SHAPE;
  if (!(tau >= 0.f && tau <= FA_MAX_RESCALE_LOG2)) return FA_ERR_SHAPE;
  if (d > 128) return FA_ERR_UNSUPPORTED;
  // N*d indexes one head with 32-bit row arithmetic; B*H*N*d*2 bytes must be addressable
  if (static_cast<int64_t>(N) * d >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t bh = static_cast<int64_t>(B) * H;
  if (bh >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t rows = bh * N;                       // < 2^62
  if (rows > (int64_t(1) << 54)) return FA_ERR_SHAPE;
  const int64_t elems = rows * d;                    // < 2^61
  const int64_t n_qt = (N + kMinBR - 1) / kMinBR;
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

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_fast(fa::Params p, hipStream_t stream) {
  static_assert(D == 64, "the 32-query kernel serves d = 64");
  constexpr int QB = FA_QB_D64;
  constexpr int BC = QB == 2 ? 32 : FA_BC_D64;
  constexpr int BR = kFNW * 32 * QB;
  p.n_qt = (p.N + BR - 1) / BR;
  const int grid = p.n_qt * p.BH;
  auto kern = fa::fa_fwd_fast_kernel<BF16, D, CAUSAL, kFNW, BC, FA_WPE_D64, false, QB>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kFNW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_wide(fa::Params p, hipStream_t stream) {
  using G = fa::WideGeom<D, FA_WIDE_BC, FA_WIDE_RING>;
  p.n_qt = (p.N + G::BR - 1) / G::BR;
  const int grid = p.n_qt * p.BH;
  auto kern = fa::fa_fwd_wide_kernel<BF16, D, CAUSAL, FA_WIDE_BC, FA_WIDE_RING>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(G::NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_generic(fa::Params p, hipStream_t stream) {
  p.n_qt = (p.N + kGBR - 1) / kGBR;
  const int grid = p.n_qt * p.BH;
  auto kern = fa::fa_fwd_generic_kernel<BF16, D, false, CAUSAL, kQB, kNW, kBC>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kNW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool BF16>
int fa_fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int N, int d, float scale, int causal, float tau, void* stream) {
  const int st = validate(q, k, v, o, lse, B, H, N, d, scale, tau);
  if (st != FA_OK) return st;

  fa::Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.N = N;
  p.d = d;
  p.BH = B * H;
  p.n_qt = 0;  // set per launch shape
  p.c = std::fabs(scale) * 1.4426950408889634f;
  p.qsign = std::signbit(scale) ? 0x80008000u : 0u;
  p.tau = tau;
  p.split_keys = 0;
  p.o_part = nullptr;
  p.l_part = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e;
  const bool cz = causal != 0;
  // scale == 0 (every allowed score equal) takes the generic kernel, which zeroes
  // masked probabilities explicitly; the fast kernel relies on exp2(-inf * c) = 0, c > 0.
  const bool fast = (d == 128 || d == 64) && p.c > 0.f;
  if (!fast) {
    if (d <= 64) e = cz ? launch_generic<BF16, 64, true>(p, s) : launch_generic<BF16, 64, false>(p, s);
    else e = cz ? launch_generic<BF16, 128, true>(p, s) : launch_generic<BF16, 128, false>(p, s);
  } else if (d == 128) {
    // 64 queries per wave, one wave per SIMD
    e = cz ? launch_wide<BF16, 128, true>(p, s) : launch_wide<BF16, 128, false>(p, s);
  } else {
    // 32 queries per wave, two or three waves per SIMD (the register count decides)
    e = cz ? launch_fast<BF16, 64, true>(p, s) : launch_fast<BF16, 64, false>(p, s);
  }
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// ---- split-KV and FA1-order passes (caller-provided workspace) --------------------
constexpr size_t kWsAlign = 256;

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Query rows per split-KV workgroup: the wide kernel's 256 at d = 128, the 32-query
// kernel's 128 at d = 64.
int split_tile(int d) {
  return d == 128 ? fa::WideGeom<128, FA_WIDE_BC, FA_WIDE_RING>::BR : kFNW * 32;
}

// Effective split count and keys per split (a multiple of the query tile), or 0.
int split_geometry(int N, int n_splits, int tile, int* keys_per_split) {
  if (N < 1 || n_splits < 1 || n_splits > FA_MAX_SPLITS) return 0;
  const int per = (N + n_splits - 1) / n_splits;
  const int keys = (per + tile - 1) / tile * tile;
  if (keys_per_split) *keys_per_split = keys;
  return (N + keys - 1) / keys;
}

size_t splitkv_bytes(int B, int H, int N, int d, int n_splits) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  const int ns = split_geometry(N, n_splits, split_tile(d), nullptr);
  if (ns == 0) return 0;
  const uint64_t rows = static_cast<uint64_t>(B) * H * N;
  if (rows > (uint64_t(1) << 40)) return 0;
  return align_up(static_cast<size_t>(ns) * rows * d * 4) + align_up(static_cast<size_t>(ns) * rows * 4);
}

size_t fa1_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  const uint64_t rows = static_cast<uint64_t>(B) * H * N;
  if (rows > (uint64_t(1) << 40)) return 0;
  return align_up(rows * d * 4) + 2 * align_up(rows * 4);
}

// Checks shared by the workspace passes, after validate(): d in {64, 128}, a nonzero
// scale, a workspace that is large enough, 256-byte aligned and disjoint from the
// tensors.
int validate_ws(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* ws, size_t ws_bytes, size_t need, int B, int H, int N, int d,
                float scale) {
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (scale == 0.f) return FA_ERR_SHAPE;
  if (!ws) return FA_ERR_NULL;
  if (need == 0 || ws_bytes < need) return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kWsAlign - 1)) != 0) return FA_ERR_ALIGN;
  const uint64_t rows = static_cast<uint64_t>(B) * H * N;
  const uint64_t tb = rows * d * 2, lb = rows * 4;
  if (ranges_overlap(ws, need, q, tb) || ranges_overlap(ws, need, k, tb) ||
      ranges_overlap(ws, need, v, tb) || ranges_overlap(ws, need, o, tb) ||
      ranges_overlap(ws, need, lse, lb))
    return FA_ERR_ALIAS;
  return FA_OK;
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_splitkv(fa::Params p, int n_eff, hipStream_t stream) {
  const int tile = split_tile(D);
  p.n_qt = (p.N + tile - 1) / tile;
  const int grid = p.n_qt * p.BH * n_eff;
  if constexpr (D == 128) {
    using G = fa::WideGeom<D, FA_WIDE_BC, FA_WIDE_RING>;
    auto kern = fa::fa_fwd_wide_kernel<BF16, D, CAUSAL, FA_WIDE_BC, FA_WIDE_RING, true>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(G::NW * 64), 0, stream, p);
  } else {
    auto kern = fa::fa_fwd_fast_kernel<BF16, D, CAUSAL, kFNW, FA_BC_D64, FA_WPE_D64, true>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kFNW * 64), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = static_cast<long long>(p.BH) * p.N;
  const long long blocks = (rows + 15) / 16;
  hipLaunchKernelGGL((fa::fa_split_merge_kernel<BF16, D>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, stream, p.o_part, p.l_part, p.o, p.lse, rows, n_eff);
  return hipGetLastError();
}

template <bool BF16>
int fa_splitkv_impl(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                    size_t ws_bytes, int B, int H, int N, int d, float scale, int causal,
                    int n_splits, void* stream) {
  int st = validate(q, k, v, o, lse, B, H, N, d, scale, 0.f);
  if (st != FA_OK) return st;
  int keys = 0;
  const int tile = split_tile(d);
  const int n_eff = split_geometry(N, n_splits, tile, &keys);
  if (n_eff == 0) return FA_ERR_SHAPE;
  const size_t need = splitkv_bytes(B, H, N, d, n_splits);
  st = validate_ws(q, k, v, o, lse, ws, ws_bytes, need, B, H, N, d, scale);
  if (st != FA_OK) return st;
  const int64_t grid = static_cast<int64_t>((N + tile - 1) / tile) * B * H * n_eff;
  if (grid >= (int64_t(1) << 31) / 64) return FA_ERR_SHAPE;
  fa::Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.N = N;
  p.d = d;
  p.BH = B * H;
  p.c = std::fabs(scale) * 1.4426950408889634f;
  p.qsign = std::signbit(scale) ? 0x80008000u : 0u;
  p.tau = FA_DEFAULT_RESCALE_LOG2;
  p.split_keys = keys;
  const uint64_t rows = static_cast<uint64_t>(p.BH) * N;
  p.o_part = static_cast<float*>(ws);
  p.l_part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                      align_up(static_cast<size_t>(n_eff) * rows * d * 4));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  hipError_t e;
  if (d == 128) e = cz ? launch_splitkv<BF16, 128, true>(p, n_eff, s) : launch_splitkv<BF16, 128, false>(p, n_eff, s);
  else e = cz ? launch_splitkv<BF16, 64, true>(p, n_eff, s) : launch_splitkv<BF16, 64, false>(p, n_eff, s);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// ---- split-KV on the library's own scratch (for callers that cannot allocate) ---------
// The partials of fa_fwd_splitkv_static live in this file-scope device array; each GPU
// holds its own copy from the code object's load until the process ends. In host code
// `scratch` only names a host-side stand-in: kernels get the device address looked up
// below, never the name.
static __device__ __align__(256) unsigned char scratch[FA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[kMaxDevices];

// Device address of the current device's `scratch`, looked up once per device with that
// device current (the first call on it) and kept for later calls.
int static_scratch(void** out) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  ScratchAddr& a = g_scratch[dev];
  std::call_once(a.once, [&a]() {
    void* ptr = nullptr;
    a.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    a.ptr = a.err == hipSuccess ? ptr : nullptr;
  });
  if (a.err != hipSuccess || a.ptr == nullptr) {
    g_last_hip_error = static_cast<int>(a.err != hipSuccess ? a.err : hipErrorInvalidSymbol);
    return FA_ERR_HIP;
  }
  *out = a.ptr;
  return FA_OK;
}

template <bool BF16>
int fa_fa1_impl(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                size_t ws_bytes, int B, int H, int N, int d, float scale, int causal, void* stream) {
  int st = validate(q, k, v, o, lse, B, H, N, d, scale, 0.f);
  if (st != FA_OK) return st;
  const size_t need = fa1_bytes(B, H, N, d);
  st = validate_ws(q, k, v, o, lse, ws, ws_bytes, need, B, H, N, d, scale);
  if (st != FA_OK) return st;
  fa::Fa1Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  const uint64_t rows = static_cast<uint64_t>(B) * H * N;
  char* w = static_cast<char*>(ws);
  p.o_ws = reinterpret_cast<float*>(w);
  p.m_ws = reinterpret_cast<float*>(w + align_up(rows * d * 4));
  p.l_ws = reinterpret_cast<float*>(w + align_up(rows * d * 4) + align_up(rows * 4));
  p.N = N;
  p.c = scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  const dim3 grid(static_cast<unsigned>(B * H)), block(256);
  if (d == 128) {
    if (cz) hipLaunchKernelGGL((fa::fa_fwd_fa1_kernel<BF16, 128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fa::fa_fwd_fa1_kernel<BF16, 128, false>), grid, block, 0, s, p);
  } else {
    if (cz) hipLaunchKernelGGL((fa::fa_fwd_fa1_kernel<BF16, 64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fa::fa_fwd_fa1_kernel<BF16, 64, false>), grid, block, 0, s, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// ---- 8-bit (e4m3) forward --------------------------------------------------------
constexpr float kFp8Tau = 2.0f;  // probabilities <= 4 before the 2^6 scale (<= 256 < 448)
#ifndef FA_FP8_NW
#define FA_FP8_NW 4  // waves (32 queries each) per workgroup of the 8-bit kernel (8: -8..18%)
#endif

// Workgroups of equal length (no causal mask) run in rounds: with three resident per CU a
// grid of W workgroups takes ceil(W / 3C) rounds of three-way shared SIMDs, with two
// ceil(W / 2C) rounds of two-way shared ones (C = CU count). When the second is shorter
// (e.g. W = 4C: 2 rounds at two per CU against 1.33, i.e. 2, rounds at three with the
// last one a third full), unused dynamic LDS caps residency at two workgroups per CU.
// The 1.15 is the measured throughput gain of the third resident workgroup.
size_t fp8_lds_cap(int grid, bool causal, size_t static_lds) {
  const int cus = fa_host::cu_count();
  const size_t per_cu = fa_host::lds_per_cu();
  if (causal || cus <= 0 || per_cu == 0 || FA_FP8_NW != 4) return 0;
  const double r3 = std::ceil(grid / (3.0 * cus)) * 3.0 / 1.15;
  const double r2 = std::ceil(grid / (2.0 * cus)) * 2.0;
  if (r2 >= r3) return 0;
  const size_t want = per_cu / 2 - 1024;  // two workgroups fit in a CU's LDS, three do not
  if (3 * want <= per_cu || want <= static_lds) return 0;
  return want - static_lds;
}

template <int D, bool CAUSAL>
hipError_t launch_fp8(fa::Fp8Params p, hipStream_t stream) {
  constexpr int BR = FA_FP8_NW * 32;
  p.n_qt = (p.N + BR - 1) / BR;
  const int grid = p.n_qt * p.BH;
  const size_t static_lds = 2 * 2 * 64 * D;  // two K and two V tiles of 64 rows
  const size_t dyn = fp8_lds_cap(grid, CAUSAL, static_lds);
  hipLaunchKernelGGL((fa::fa_fwd_fp8_kernel<D, CAUSAL, FA_FP8_NW>), dim3(grid),
                     dim3(FA_FP8_NW * 64), dyn, stream, p);
  return hipGetLastError();
}

int fa_fp8_impl(const void* q, const void* k, const void* v, float q_scale, float k_scale,
                float v_scale, void* o, float* lse, int B, int H, int N, int d, float scale,
                int causal, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_SHAPE;
  if (!std::isfinite(scale) || !std::isfinite(q_scale) || !std::isfinite(k_scale) ||
      !std::isfinite(v_scale))
    return FA_ERR_SHAPE;
  const double cs = static_cast<double>(scale) * q_scale * k_scale;
  if (cs == 0.0 || !std::isfinite(cs) || std::fabs(cs) * 1.4426950408889634 > 3.0e38)
    return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(N) * d >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t bh = static_cast<int64_t>(B) * H;
  if (bh >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  const int64_t rows = bh * N;
  if (rows > (int64_t(1) << 54)) return FA_ERR_SHAPE;
  if (((N + 127) / 128) * bh >= (int64_t(1) << 31) / 64) return FA_ERR_SHAPE;
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if ((a16 & 15u) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_ALIGN;
  const uint64_t ib = static_cast<uint64_t>(rows) * d, ob = ib * 2, lb = rows * 4;
  if (ranges_overlap(o, ob, q, ib) || ranges_overlap(o, ob, k, ib) || ranges_overlap(o, ob, v, ib) ||
      ranges_overlap(lse, lb, q, ib) || ranges_overlap(lse, lb, k, ib) ||
      ranges_overlap(lse, lb, v, ib) || ranges_overlap(lse, lb, o, ob))
    return FA_ERR_ALIAS;
  fa::Fp8Params p;
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.N = N;
  p.BH = static_cast<int>(bh);
  p.n_qt = 0;
  p.c = static_cast<float>(std::fabs(cs) * 1.4426950408889634);
  p.qsign = cs < 0.0 ? 0x80808080u : 0u;
  p.vs = v_scale;
  p.tau = kFp8Tau;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  hipError_t e;
  if (d == 128) e = cz ? launch_fp8<128, true>(p, s) : launch_fp8<128, false>(p, s);
  else e = cz ? launch_fp8<64, true>(p, s) : launch_fp8<64, false>(p, s);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
               float v_scale, void* o, float* lse, int B, int H, int N, int d, float scale,
               int causal, void* stream) {
  return fa_fp8_impl(q, k, v, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale, causal,
                     stream);
}


size_t fa_fwd_splitkv_workspace_size(int B, int H, int N, int d, int n_splits) {
  return splitkv_bytes(B, H, N, d, n_splits);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   float scale, int causal, int n_splits, int dtype, void* stream) {
  if (dtype == FA_DTYPE_BF16)
    return fa_splitkv_impl<true>(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale,
                                 causal, n_splits, stream);
  if (dtype == FA_DTYPE_FP16)
    return fa_splitkv_impl<false>(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale,
                                  causal, n_splits, stream);
  return FA_ERR_UNSUPPORTED;
}

int fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, int n_splits,
                          int dtype, void* stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return FA_ERR_UNSUPPORTED;
  // the checks of fa_fwd_splitkv that do not involve the workspace, before any HIP call
  int st = validate(q, k, v, o, lse, B, H, N, d, scale, 0.f);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (scale == 0.f) return FA_ERR_SHAPE;
  const size_t need = splitkv_bytes(B, H, N, d, n_splits);
  if (need == 0) return FA_ERR_SHAPE;
  if (need > FA_STATIC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != FA_OK) return st;
  if (dtype == FA_DTYPE_BF16)
    return fa_splitkv_impl<true>(q, k, v, o, lse, ws, FA_STATIC_SCRATCH_BYTES, B, H, N, d,
                                 scale, causal, n_splits, stream);
  return fa_splitkv_impl<false>(q, k, v, o, lse, ws, FA_STATIC_SCRATCH_BYTES, B, H, N, d,
                                scale, causal, n_splits, stream);
}

size_t fa_fwd_fa1_workspace_size(int B, int H, int N, int d) { return fa1_bytes(B, H, N, d); }

int fa_fwd_fa1(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
               size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
               int dtype, void* stream) {
  if (dtype == FA_DTYPE_BF16)
    return fa_fa1_impl<true>(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale,
                             causal, stream);
  if (dtype == FA_DTYPE_FP16)
    return fa_fa1_impl<false>(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale,
                              causal, stream);
  return FA_ERR_UNSUPPORTED;
}


int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, void* stream) {
  return fa_fwd_impl<true>(q, k, v, o, lse, B, H, N, d, scale, causal,
                           FA_DEFAULT_RESCALE_LOG2, stream);
}

int fa_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int N, int d, float scale, int causal, void* stream) {
  return fa_fwd_impl<false>(q, k, v, o, lse, B, H, N, d, scale, causal,
                            FA_DEFAULT_RESCALE_LOG2, stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int N, int d, float scale, int causal, int dtype, float rescale_log2,
              void* stream) {
  if (dtype == FA_DTYPE_BF16)
    return fa_fwd_impl<true>(q, k, v, o, lse, B, H, N, d, scale, causal, rescale_log2, stream);
  if (dtype == FA_DTYPE_FP16)
    return fa_fwd_impl<false>(q, k, v, o, lse, B, H, N, d, scale, causal, rescale_log2, stream);
  return FA_ERR_UNSUPPORTED;
}

int fa_fwd_supported(int d, int dtype, int causal) {
  (void)causal;
  if (d < 1 || d > 128) return 0;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP16) return 0;
  return 1;
}

int fa_device_supported(int device) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) {
    (void)hipGetLastError();  // leave no sticky error behind
    return 0;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

int fa_device_info(int device, int* cu_count, int* clock_khz) {
  if (cu_count == nullptr || clock_khz == nullptr) return FA_ERR_NULL;
  *cu_count = 0;
  *clock_khz = 0;
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e == hipSuccess && (device < 0 || device >= n)) e = hipErrorInvalidDevice;
  hipDeviceProp_t prop;
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // leave no sticky error behind
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
  }
  *cu_count = prop.multiProcessorCount;
  *clock_khz = prop.clockRate;
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape, scale or rescale threshold (B, H, N, d >= 1; finite scale; 0 <= threshold <= 15; sizes in range)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (1 <= d <= 128) or dtype";
    case FA_ERR_ALIAS: return "o or lse overlaps q, k, v or each other";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_HIP: return "the HIP runtime refused the launch (see fa_last_hip_error)";
    case FA_ERR_SCRATCH: return "split-KV partials exceed the library's static scratch (FA_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

const char* fa_version(void) {
  return "fa355 0.2.0 (gfx950: FA2-order forward bf16/fp16/fp8, backward, split-KV, FA1 ablation)";
}

}  // extern "C"
