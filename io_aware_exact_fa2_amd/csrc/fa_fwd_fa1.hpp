// fa_fwd_fa1.hpp — the FA1 loop order, as an ablation of the FA2-order kernels (gfx950).
//
// [P1] currybab.bearblog.dev, "FlashAttention 1 forward pass 알고리즘 분석" and the
// "정리" comparison table: the key/value block K_j, V_j is the outer loop and every
// query block Q_i the inner loop; per block the kernel computes S_ij = Q_i K_j^T, the
// block statistics m~_ij (row max), P~_ij = exp(S_ij - m~_ij) and l~_ij (row sum), and
// merges them with the running m_i, l_i read back from device memory:
//     m_new = max(m_i, m~_ij),  alpha = exp(m_i - m_new),  beta = exp(m~_ij - m_new),
//     l_new = alpha l_i + beta l~_ij,
//     O_i  <- (l_i alpha O_i + beta P~_ij V_j) / l_new      (O_i kept normalized),
// then writes O_i, m_i, l_i back. The work is parallel over (batch, head) only, as in
// the table ("병렬화 단위"); each workgroup walks all blocks of its head in order.
// Per head this moves Q T_c times and O_i through device memory 2 (T_c - 1) times,
// the table's HBM column, where the FA2-order kernels read Q once and write O once.
//
// Readings: the running O_i, m_i and l_i live in a float32 workspace (16-bit storage of
// O_i would add T_c roundings); the first key block initialises the state instead of
// reading it (m = -inf, l = 0, O = 0 give the same update), and the last block a row
// block visits writes the final O (16-bit) and L = m + log l instead of the workspace.
// The products run on the same MFMA layouts as the FA2-order kernels (S^T = K Q^T with
// the query on the lane, O^T = V^T P^T).
#pragma once

#include "fa_common.hpp"

namespace fa {

struct Fa1Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* o_ws;  // [BH, N, D] running normalized O_i
  float* m_ws;  // [BH, N] running max, log2 units
  float* l_ws;  // [BH, N] running sum
  int N;
  float c;  // scale * log2(e), signed
};

template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fa_fwd_fa1_kernel(const Fa1Params p) {
  using E = Elt<BF16>;
  constexpr int NW = 4, BC = 64, BRI = NW * 32, CPR = D / 8, NDS = D / 16;
  __shared__ __attribute__((aligned(1024))) u32x4_t ks[BC * CPR];
  __shared__ __attribute__((aligned(1024))) u32x4_t vs[BC * CPR];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int N = p.N, bh = blockIdx.x;
  const size_t head = (size_t)bh * (size_t)N * D;
  const int T_c = (N + BC - 1) / BC, T_r = (N + BRI - 1) / BRI;
  constexpr float kLn2 = 0.69314718055994530942f;

  // LDS operand addresses: K rows (A of S^T, row rho(m) at MFMA row m) and V^T
  // (transposed reads), with the swizzles of the FA2-order kernels
  int kaddr[NDS], vaddr[D / 32];
  {
    const int row = key_of_row(l32);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kaddr[ds] = (row * CPR + ((2 * ds + hh) ^ swz_k<D>(row))) * 16;
    const int g16 = lane >> 4, t4 = (lane & 15) >> 2, u4 = lane & 3;
    const int vrow = (g16 >> 1) * 8 + t4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vaddr[db] = (vrow * CPR + ((4 * db + 2 * (g16 & 1) + (u4 >> 1)) ^ swz_v<D>(vrow))) * 16 +
                  (u4 & 1) * 8;
  }
  auto k_frag = [&](int kb, int ds) {
    return *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const unsigned char*>(ks) +
                                             kaddr[ds] + kb * 32 * CPR * 16);
  };
  auto v_frag = [&](int db, int st) {
    const unsigned char* b = reinterpret_cast<const unsigned char*>(vs) + vaddr[db];
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b + (16 * st) * CPR * 16));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b + (16 * st + 4) * CPR * 16));
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };

  for (int j = 0; j < T_c; ++j) {
    const int k0 = j * BC;
    __syncthreads();  // the previous block's reads are done
#pragma unroll
    for (int t = 0; t < BC * CPR / 256; ++t) {
      const int idx = tid + 256 * t, row = idx / CPR, ch = idx % CPR;
      u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (k0 + row < N) {
        kx = ld16(p.k + head + (size_t)(k0 + row) * D + ch * 8);
        vx = ld16(p.v + head + (size_t)(k0 + row) * D + ch * 8);
      }
      ks[row * CPR + (ch ^ swz_k<D>(row))] = kx;
      vs[row * CPR + (ch ^ swz_v<D>(row))] = vx;
    }
    __syncthreads();
    // query blocks whose rows all precede the key block see none of its keys
    for (int i = CAUSAL ? k0 / BRI : 0; i < T_r; ++i) {
      const int wq0 = i * BRI + wid * 32;
      if (wq0 >= N || (CAUSAL && wq0 + 31 < k0)) continue;
      const int qi = wq0 + l32, qr = min(qi, N - 1);
      const int w_last = CAUSAL ? min(T_c - 1, min(wq0 + 31, N - 1) / BC) : T_c - 1;
      // S^T of the 64 keys x 32 queries, in log2 units, masked entries -inf
      u32x4_t qf[NDS];
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) qf[ds] = ld16(p.q + head + (size_t)qr * D + ds * 16 + hh * 8);
      f32x16_t s[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) s[kb] = E::mfma(k_frag(kb, ds), qf[ds], s[kb]);
      }
      float mt = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + key_of_reg(r, hh);
          float t = s[kb][r] * p.c;
          if (key >= N || (CAUSAL && key > qi)) t = -__builtin_inff();
          s[kb][r] = t;
          mt = __builtin_fmaxf(mt, t);
        }
      mt = xhalf_max(mt);  // m~_ij; -inf when the row sees no key of this block
      // P~ = exp(S - m~), l~ = rowsum P~ (both 0 for a row with no key here)
      const float msub = mt == -__builtin_inff() ? 0.f : mt;
      u32x4_t pb[BC / 16];
      float lt = 0.f;
#pragma unroll
      for (int e = 0; e < BC / 2; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[e / 16][e % 16] - msub);
        const float p1 = __builtin_amdgcn_exp2f(s[e / 16][(e + 1) % 16] - msub);
        lt += p0 + p1;
        pb[e / 8][(e % 8) / 2] = E::pack(p0, p1);
      }
      lt = xhalf_sum(lt);
      // P~ V_j (O^T layout: lane = query, registers = head dims)
      f32x16_t pv[D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[db][r] = 0.f;
#pragma unroll
        for (int st = 0; st < BC / 16; ++st) pv[db] = E::mfma(v_frag(db, st), pb[st], pv[db]);
      }
      // merge with the running statistics of the row
      const size_t srow = (size_t)bh * N + qr;
      float mi = -__builtin_inff(), li = 0.f;
      if (j > 0) {
        mi = p.m_ws[srow];
        li = p.l_ws[srow];
      }
      const float mnew = __builtin_fmaxf(mi, mt);  // finite: block 0 holds key 0
      const float alpha = __builtin_amdgcn_exp2f(mi - mnew);
      const float beta = __builtin_amdgcn_exp2f(mt - mnew);
      const float lnew = alpha * li + beta * lt;
      const float a = li * alpha / lnew, b = beta / lnew;
      float* orow = p.o_ws + srow * D;
      const bool last = j == w_last;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dcol = db * 32 + g * 8 + hh * 4;
          float4 oi = float4{0.f, 0.f, 0.f, 0.f};
          if (j > 0) oi = *reinterpret_cast<const float4*>(orow + dcol);
          const float4 on = float4{a * oi.x + b * pv[db][4 * g], a * oi.y + b * pv[db][4 * g + 1],
                                   a * oi.z + b * pv[db][4 * g + 2], a * oi.w + b * pv[db][4 * g + 3]};
          if (qi < N) {
            if (last)
              *reinterpret_cast<u32x2_t*>(p.o + head + (size_t)qi * D + dcol) =
                  u32x2_t{E::pack(on.x, on.y), E::pack(on.z, on.w)};
            else
              *reinterpret_cast<float4*>(orow + dcol) = on;
          }
        }
      if (qi < N && hh == 0) {
        if (last) {
          p.lse[srow] = (mnew + __builtin_amdgcn_logf(lnew)) * kLn2;
        } else {
          p.m_ws[srow] = mnew;
          p.l_ws[srow] = lnew;
        }
      }
    }
  }
}

}  // namespace fa
