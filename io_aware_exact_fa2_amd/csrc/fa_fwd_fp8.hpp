// fa_fwd_fp8.hpp — FA2-order attention forward with 8-bit (OCP e4m3) Q, K, V (gfx950).
//
// The FA2 loop order of [P1] currybab.bearblog.dev ("FlashAttention 2 forward pass 알고리즘
// 분석"), on the 8-bit matrix cores that the FP8 path of [P2] iq-universe.github.io ("v2와
// v3": FP8 doubles the matrix throughput over 16-bit inputs) refers to:
//   * Q, K, V are e4m3 with one float scale per tensor (value = code * scale); the scores
//     are S = scale * qs * ks * (Q8 K8^T), accumulated in fp32 by
//     v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales);
//   * the online softmax (running max, rescale by alpha, sum l) runs in fp32 as in the
//     16-bit kernels; a row's reference max is raised only when a block's max exceeds it
//     by more than tau = 2 (log2 units), so the unnormalised probabilities stay at or
//     below 4; they are scaled by 2^6 (folded into the exponent; the factor cancels
//     between O and l) and rounded to e4m3 for the P V product: at most 256 < 448, the
//     largest e4m3 value, and normal (3 mantissa bits) down to 2^-12 of the reference,
//     where the format's subnormal range begins. l sums them unrounded;
//   * O = vs * (P8 V8) / l is written as bfloat16, L as float32.
// Layouts: S^T = K Q^T with the query on the lane. MFMA row m of key block kb reads key
// 32 ((m >> 2) & 1) + 16 kb + 4 (m >> 3) + (m & 3), so the 16 accumulators of lane half h
// in block kb hold keys 32 h + 16 kb + r (r = 0..15): packed to bytes, the two blocks are
// exactly the 32 consecutive keys that lane half h supplies as the B operand of the
// 64-key P V product. V^T operands are read with ds_read_b64_tr_b8 (each lane of a
// 16-lane group receives one column of 8 rows). Tiles go HBM -> LDS by buffer-to-LDS
// copies into two buffers, the next tile's copies in flight while the current one is
// computed (one barrier per tile). Workgroups of NW waves of 32 queries each (4 by
// default: three workgroups share a CU at d = 128).
#pragma once

#include "fa_common.hpp"

namespace fa {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;  // bfloat16
  float* lse;
  int N;
  int BH;
  int n_qt;
  float c;        // |scale * qs * ks| * log2(e)
  uint32_t qsign; // 0x80808080 when scale * qs * ks < 0 (Q negated on load), else 0
  float vs;       // V scale
  float tau;      // rescale threshold, log2 units (at most 2: P' = 2^6 P stays <= 256)
};

// Chunk swizzles (16-byte chunks, rows of D bytes). K rows are read as MFMA row operands
// (a quarter-wave reads one logical chunk of 16 rows: two runs of 8 consecutive rows 32
// apart); V rows with ds_read_b64_tr_b8 (a half-wave reads 8 consecutive rows x 2
// chunks). Each swizzle maps those rows to distinct 16-byte bank granules.
template <int D> __device__ __forceinline__ int swz8_k(int row) {
  return D == 128 ? (((row >> 1) & 3) | (((row >> 5) & 1) << 2))
                  : (((row >> 2) & 1) | (((row >> 5) & 1) << 1));
}
template <int D> __device__ __forceinline__ int swz8_v(int row) {
  return D == 128 ? 2 * ((row >> 1) & 3) : 2 * ((row >> 2) & 1);
}

#ifndef FA_FP8_WPE
#define FA_FP8_WPE 2  // least waves per SIMD the register budget must allow
#endif

template <int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FA_FP8_WPE)))
fa_fwd_fp8_kernel(const Fp8Params p) {
  constexpr int BR = NW * 32, BC = 64, CPR = D / 16;  // 16-byte chunks per row
  constexpr int NT = D / 64;                                  // 64-deep MFMA steps over d
  constexpr int TOT = BC * CPR;                               // chunks per tile and tensor
  static_assert(D == 64 || D == 128, "head dims");
  __shared__ __attribute__((aligned(1024))) u32x4_t ks2[2][BC * CPR];
  __shared__ __attribute__((aligned(1024))) u32x4_t vs2[2][BC * CPR];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N;
  int bh, qt;
  tile_order<CAUSAL>(blockIdx.x, p.BH, p.n_qt, bh, qt);
  if (CAUSAL) qt = p.n_qt - 1 - qt;  // the last query tile sees the most keys
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint8_t* __restrict__ kg = p.k + head;
  const uint8_t* __restrict__ vg = p.v + head;
  const int q0 = qt * BR, wq0 = q0 + wid * 32;
  const int q_end = min(q0 + BR, N);
  const int n_kt = CAUSAL ? (q_end + BC - 1) / BC : (N + BC - 1) / BC;
  const bool wave_live = wq0 < N;
  const int w_last_q = min(wq0 + 32, N) - 1;
  const int w_kt = CAUSAL ? min(n_kt, w_last_q / BC + 1) : n_kt;
  const int qi = wq0 + l32;

  // Q as the B operand of S^T: lane (query qi, half hh) holds d = 64 t + 32 hh .. + 31
  i32x8_t qf[NT];
  {
    const int qr = min(qi, N - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint8_t* src = p.q + head + (size_t)qr * D + 64 * t + 32 * hh;
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(src);
      const u32x4_t b = *reinterpret_cast<const u32x4_t*>(src + 16);
      qf[t] = i32x8_t{(int)(a[0] ^ p.qsign), (int)(a[1] ^ p.qsign), (int)(a[2] ^ p.qsign),
                      (int)(a[3] ^ p.qsign), (int)(b[0] ^ p.qsign), (int)(b[1] ^ p.qsign),
                      (int)(b[2] ^ p.qsign), (int)(b[3] ^ p.qsign)};
    }
  }

  // LDS read addresses. K: block kb, MFMA row m = l32 -> key row krow(kb); the chunks
  // 4 t + 2 hh and 4 t + 2 hh + 1 (d = 64 t + 32 hh .. + 31).
  auto krow = [&](int kb) { return 32 * ((l32 >> 2) & 1) + 16 * kb + 4 * (l32 >> 3) + (l32 & 3); };
  auto k_op = [&](const u32x4_t* ks, int kb, int t) {
    const int row = krow(kb);
    const u32x4_t a = ks[row * CPR + ((4 * t + 2 * hh) ^ swz8_k<D>(row))];
    const u32x4_t b = ks[row * CPR + ((4 * t + 2 * hh + 1) ^ swz8_k<D>(row))];
    return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                   (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  };
  // V^T operand of d block db: lane (group g16: column 32 db + 16 (g16 & 1) + i, keys
  // 32 (g16 >> 1) + 8 j .. + 7 for j = 0..3). In the group, lane (t8, u2) supplies row
  // 32 (g16 >> 1) + 8 j + t8, bytes 8 u2 .. 8 u2 + 7 of chunk 2 db + (g16 & 1).
  const int g16 = lane >> 4, t8 = (lane & 15) >> 1, u2 = lane & 1;
  auto v_op = [&](const u32x4_t* vs, int db) {
    i32x8_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 32 * (g16 >> 1) + 8 * j + t8;
      const int ch = (2 * db + (g16 & 1)) ^ swz8_v<D>(row);
      const unsigned char* b = reinterpret_cast<const unsigned char*>(vs) + (row * CPR + ch) * 16 + 8 * u2;
      const i32x2_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)b);
      r[2 * j] = x[0];
      r[2 * j + 1] = x[1];
    }
    return r;
  };

  // Tiles go HBM -> LDS by buffer loads with an LDS destination (no register staging).
  // Each wave copies whole 1 KB pieces: lane l of copy c writes chunk (wid + NW c) * 64 + l
  // of the tile and fetches the logical chunk that the tensor's swizzle puts there. The
  // buffer range ends at key N, so rows past N read as zero bytes (+0 in E4M3; their
  // scores are masked to -inf, so their probabilities are 0).
  constexpr int PERW = TOT / (64 * NW);
  static_assert(TOT % (64 * NW) == 0, "whole 1 KB copies per wave");
  int koff[PERW], voff[PERW];
#pragma unroll
  for (int cc = 0; cc < PERW; ++cc) {
    const int f = (wid + NW * cc) * 64 + lane, row = f / CPR, ph = f % CPR;
    koff[cc] = row * D + (ph ^ swz8_k<D>(row)) * 16;
    voff[cc] = row * D + (ph ^ swz8_v<D>(row)) * 16;
  }
  auto issue = [&](int j, u32x4_t* kdst, u32x4_t* vdst) {
    const int k0 = j * BC;
    const int bytes = min(N - k0, BC) * D;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kg + (size_t)k0 * D), (short)0, bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(vg + (size_t)k0 * D), (short)0, bytes, kBufferWord3);
    // (destinations and offsets are arguments: a lambda that captured the shared arrays
    // or the offset arrays here made the host pass drop the kernel's launch stub; wid is
    // wave-uniform, read from the first lane, as the LDS destination base must be)
    auto copy = [&](int cc, int ko, int vo) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + (wid + NW * cc) * 64), 16,
                                               ko, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + (wid + NW * cc) * 64), 16,
                                               vo, 0, 0, 0);
    };
#pragma unroll
    for (int cc = 0; cc < PERW; ++cc) copy(cc, koff[cc], voff[cc]);
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float ms = -__builtin_inff(), l_part = 0.f;
  const float c = p.c;

  // Tile t lives in buffer t % 2. Iteration j issues the copies of tile j+1 into the
  // other buffer, whose last readers (tile j-1) all passed the previous barrier, computes
  // tile j, waits for its own copies and meets one barrier.
  issue(0, ks2[0], vs2[0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int j = 0; j < n_kt; ++j) {
    const int k0 = j * BC;
    if (j + 1 < n_kt) issue(j + 1, ks2[(j + 1) & 1], vs2[(j + 1) & 1]);
    const u32x4_t* ks = ks2[j & 1];
    const u32x4_t* vs = vs2[j & 1];
    if (wave_live && j < w_kt) {
      // S^T of the 64 keys (two 32-key blocks)
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k_op(ks, kb, t), qf[t], s[kb], 0, 0, 0,
                                                                  0, 0, 0);
      }
      // masks on the tiles that reach past N or cross the diagonal
      if (k0 + BC > N || (CAUSAL && k0 + BC - 1 > wq0)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * hh + 16 * kb + r;
            if (key >= N || (CAUSAL && key > qi)) s[kb][r] = -__builtin_inff();
          }
      }
      // running max (raw dot units); rescale only when some row rose by more than tau
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][r]);
      mx = xhalf_max(mx) * c;
      if (__builtin_amdgcn_ballot_w64(mx > ms + p.tau) != 0) {
        const float ms_new = __builtin_fmaxf(ms, mx);
        const float alpha = __builtin_amdgcn_exp2f(ms - ms_new);  // 0 on the first tile
        ms = ms_new;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      // P' = 2^6 exp2(s c - m) <= 256: fp32 sum, e4m3 bytes for the P V product (key
      // 32 hh + 16 kb + r is byte 16 kb + r of the lane's operand)
      i32x8_t pb;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float pv[4];
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            pv[y] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * w + y], c, 6.0f - ms));
            l_part += pv[y];
          }
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], word, true);
          pb[4 * kb + w] = word;
        }
      // O^T += V^T P^T over the 64 keys
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v_op(vs, db), pb, oacc[db], 0, 0, 0,
                                                                   0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile j+1's copies
    __syncthreads();
  }

  // epilogue: O = vs * O~ / l (bfloat16; the 2^6 cancels), L = (m - 6 + log2 l) ln 2
  if (!wave_live || qi >= N) return;
  const float l_tot = xhalf_sum(l_part);
  const float mul = p.vs / l_tot;
  uint16_t* orow = p.o + head + (size_t)qi * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = db * 32 + g * 8 + hh * 4;
      const f32x16_t& a = oacc[db];
      *reinterpret_cast<u32x2_t*>(orow + dcol) =
          u32x2_t{Elt<true>::pack(a[4 * g] * mul, a[4 * g + 1] * mul),
                  Elt<true>::pack(a[4 * g + 2] * mul, a[4 * g + 3] * mul)};
    }
  if (hh == 0)
    p.lse[(size_t)bh * N + qi] = (ms - 6.0f + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
}

}  // namespace fa
