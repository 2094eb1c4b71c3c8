// fa_fwd_generic.hpp — FA2-order attention forward for gfx950 (MI355X): the generic
// kernel, used for head dims other than 64 and 128 (bounds-checked, zero-filled columns).
//
// Algorithm ([P1] currybab.bearblog.dev, "Triton으로 FlashAttention 구현하기 전에 -
// FA1, 2 forward pass", section "FlashAttention 2 forward pass 알고리즘 분석"):
// one workgroup owns a block of query rows (outer loop) and streams the key/value
// blocks through LDS (inner loop). Per key block, for each of its rows:
//     S = Q_i K_j^T,  m_new = max(m_old, rowmax S),  P~ = exp(S - m_new),
//     l = alpha*l + rowsum(P~),  O~ = alpha*O~ + P~ V_j,  alpha = exp(m_old - m_new);
// after the last block O = O~ / l and L = m + log l (the section's per-block update
// and epilogue equations). Work is split over workgroups by (query block, head, batch)
// — the sequence parallelism of that section — and inside a workgroup every wave
// owns its own query rows (split-Q), so no cross-wave merge exists.
//
// gfx950 mapping
//   * Both contractions run on v_mfma_f32_32x32x16_{bf16,f16}. The kernel computes
//     S^T = K Q^T and O^T = V^T P^T so that each lane owns ONE query column: the
//     row max, row sum and the alpha rescale of O~ are then in-lane, and the fp32
//     S^T accumulator, rounded to 16 bits, is already the B operand of the P V
//     MFMA (no LDS round trip for P).
//   * Key rows are placed in the S^T MFMA with bits 2 and 3 of the row index
//     swapped. The accumulator register r of lane-half h then holds key
//     r + 8h + (r & 8) of the 32-key block, so each lane's 8 values for one 16-key
//     step of P V are 8 consecutive keys and V^T is read with one 16-byte LDS load.
//   * K is staged row-major in LDS with a 16-byte row pad; V is staged transposed
//     (V^T, 16-byte key units XOR-swizzled by the row) so both MFMA A operands are
//     single ds_read_b128 loads without bank conflicts.
//   * Global loads are 16 bytes per lane, issued one tile ahead into registers
//     and written to the other half of a double-buffered LDS stage: one barrier
//     per key tile.
//   * Scores are never scaled: exp2(s*c - m*c) with c = |scale|*log2(e) costs one
//     FMA and one v_exp_f32 per score; the running max is kept in raw units.
//   * Causal: key tiles whose first key is past the workgroup's last query are
//     never loaded ([P2] iq-universe.github.io, "FlashAttention은 어떻게 O(N²)
//     메모리 벽을 넘었나", section "v2와 v3": whole blocks above the diagonal are
//     skipped); a wave also skips tiles past its own last query; element masks are
//     applied only on diagonal and ragged-tail tiles.
#pragma once

#include "fa_common.hpp"

namespace fa {

// --- tile geometry ----------------------------------------------------------------
template <int D_, int QB_, int NW_, int BC_>
struct GenericGeom {
  static constexpr int D = D_;      // padded head dim: 64 or 128
  static constexpr int QB = QB_;    // 32-query blocks per wave
  static constexpr int NW = NW_;    // waves per workgroup
  static constexpr int BC = BC_;    // keys per tile
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * QB * 32;       // queries per workgroup
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int KCH = BC * CPR / NT;     // chunks per thread per tensor per tile
  static constexpr int KPITCH = D * 2 + 16;     // K row pitch in LDS (bytes)
  static constexpr int K_BYTES = BC * KPITCH;
  static constexpr int VPITCH = BC * 2;         // V^T row pitch (bytes), no pad
  static constexpr int VUNITS = BC / 8;         // 16-byte key units per V^T row
  static constexpr int VT_BYTES = D * VPITCH;
  static constexpr int STAGE = K_BYTES + VT_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static_assert(D == 64 || D == 128, "padded head dim");
  static_assert(BC == 64, "V^T swizzle is laid out for 64-key tiles");
  static_assert((BC * CPR) % NT == 0 && KCH >= 2 && KCH <= 4 && (KCH & (KCH - 1)) == 0,
                "tile loader split");
  static_assert(BC / KCH * CPR == NT, "V transposing loader covers the tile exactly");
};

// XOR swizzle of the 16-byte key units of V^T row `dcol` (conflict-free b128 reads
// along consecutive rows, at most 2-way conflicts on the b64 transposing writes).
__device__ __forceinline__ int vt_swz(int dcol) { return ((dcol >> 1) ^ (dcol >> 4)) & 7; }

// Bounds-checked 8-element load for head dims that are not the padded size.
__device__ __forceinline__ u32x4_t ld8_ragged(const uint16_t* row, int col, int d) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c0 = col + 2 * i;
    const uint32_t lo = c0 < d ? row[c0] : 0u;
    const uint32_t hi = c0 + 1 < d ? row[c0 + 1] : 0u;
    w[i] = lo | (hi << 16);
  }
  return u32x4_t{w[0], w[1], w[2], w[3]};
}

template <bool BF16, int D, bool EXACT_D, bool CAUSAL, int QB, int NW, int BC>
__global__ void __launch_bounds__(NW * 64)
fa_fwd_generic_kernel(const Params p) {
  using G = GenericGeom<D, QB, NW, BC>;
  using E = Elt<BF16>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int N = p.N;
  const int dstride = EXACT_D ? D : p.d;

  // ---- workgroup -> (head, query tile) -------------------------------------------
  int bh, qt;
  decode_tile<CAUSAL>(p, blockIdx.x, bh, qt);
  const size_t head = (size_t)bh * (size_t)N * (size_t)dstride;
  const uint16_t* __restrict__ qg = p.q + head;
  const uint16_t* __restrict__ kg = p.k + head;
  const uint16_t* __restrict__ vg = p.v + head;

  const int q0 = qt * G::BR;
  const int wq0 = q0 + w * QB * 32;            // first query of this wave
  const int q_end = min(q0 + G::BR, N);        // one past the last real query of the tile
  const int n_kt = CAUSAL ? (q_end + BC - 1) / BC : (N + BC - 1) / BC;
  const bool wave_live = wq0 < N;
  const int w_last_q = min(wq0 + QB * 32, N) - 1;
  const int w_kt = CAUSAL ? min(n_kt, w_last_q / BC + 1) : n_kt;

  // ---- Q fragments: B operand of S^T = K Q^T, kept in registers -------------------
  u32x4_t qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = wq0 + qb * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const int col = ds * 16 + hh * 8;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (qi < N) {
        if (EXACT_D) x = ld16(qg + (size_t)qi * D + col);
        else x = ld8_ragged(qg + (size_t)qi * dstride, col, p.d);
      }
      qf[qb][ds] = x ^ p.qsign;
    }
  }

  // ---- tile staging: global -> registers -> LDS ------------------------------------
  u32x4_t kst[G::KCH], vst[G::KCH];
  const int v_dch = tid % G::CPR;              // V: 8 head-dim columns ...
  const int v_kg = tid / G::CPR;               // ... of KCH consecutive keys

  auto load_tile = [&](int j) {
    const int k0 = j * BC;
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      const int id = tid + i * G::NT;
      const int row = id / G::CPR, ch = id % G::CPR;
      const int key = k0 + row;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (key < N) {
        if (EXACT_D) x = ld16(kg + (size_t)key * D + ch * 8);
        else x = ld8_ragged(kg + (size_t)key * dstride, ch * 8, p.d);
      }
      kst[i] = x;
    }
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      const int key = k0 + v_kg * G::KCH + i;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (key < N) {
        if (EXACT_D) x = ld16(vg + (size_t)key * D + v_dch * 8);
        else x = ld8_ragged(vg + (size_t)key * dstride, v_dch * 8, p.d);
      }
      vst[i] = x;
    }
  };

  auto store_tile = [&](int buf) {
    unsigned char* ks = smem + buf * G::STAGE;
    unsigned char* vts = ks + G::K_BYTES;
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      const int id = tid + i * G::NT;
      const int row = id / G::CPR, ch = id % G::CPR;
      *reinterpret_cast<u32x4_t*>(ks + row * G::KPITCH + ch * 16) = kst[i];
    }
    // transpose: this thread holds keys [key0, key0+KCH) x columns [8*v_dch, 8*v_dch+8)
    const int key0 = v_kg * G::KCH;
    const int unit = key0 >> 3, in_unit = (key0 & 7) * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dcol = v_dch * 8 + e;
      const int word = e >> 1, sh = (e & 1) * 16;
      unsigned char* dst = vts + dcol * G::VPITCH + ((unit ^ vt_swz(dcol)) << 4) + in_unit;
      if constexpr (G::KCH == 4) {
        const uint32_t a0 = (vst[0][word] >> sh) & 0xffffu, a1 = (vst[1][word] >> sh) & 0xffffu;
        const uint32_t a2 = (vst[2][word] >> sh) & 0xffffu, a3 = (vst[3][word] >> sh) & 0xffffu;
        *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{a0 | (a1 << 16), a2 | (a3 << 16)};
      } else {
        const uint32_t a0 = (vst[0][word] >> sh) & 0xffffu, a1 = (vst[1][word] >> sh) & 0xffffu;
        *reinterpret_cast<uint32_t*>(dst) = a0 | (a1 << 16);
      }
    }
  };

  // ---- per-lane running state ------------------------------------------------------
  f32x16_t oacc[D / 32][QB];
  float m_run[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_part[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  }
  const float c = p.c;
  const int krow_off = key_of_row(l32) * G::KPITCH + hh * 16;
  int vrow_off[D / 32], vswz[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    vrow_off[db] = (db * 32 + l32) * G::VPITCH;
    vswz[db] = vt_swz(db * 32 + l32);
  }

  auto compute_tile = [&](int buf, int j) {
    const unsigned char* ks = smem + buf * G::STAGE;
    const unsigned char* vts = ks + G::K_BYTES;
    const int k0 = j * BC;

    // S^T = K Q^T (raw dot products)
    f32x16_t s[BC / 32][QB];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
      const unsigned char* krow = ks + kb * 32 * G::KPITCH + krow_off;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(krow + ds * 32);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = E::mfma(kf, qf[qb][ds], s[kb][qb]);
      }
    }

    // masks only on the ragged tail tile and on tiles that cross the diagonal
    const bool masked = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > wq0);
    if (masked) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qi = wq0 + qb * 32 + l32;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + key_of_reg(r, hh);
            const bool drop = key >= N || (CAUSAL && key > qi);
            if (drop) s[kb][qb][r] = -__builtin_inff();
          }
      }
    }

    // online softmax, one query per lane (two lanes per query: lane and lane^32)
    u32x4_t pb[BC / 16][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][qb][r]);
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      const float m_old = m_run[qb];
      const float m_new = __builtin_fmaxf(m_old, mx);
      const bool fresh = m_new == -__builtin_inff();    // nothing allowed seen yet
      const float msc = fresh ? 0.f : m_new * c;
      const float alpha = (m_old == -__builtin_inff()) ? 0.f
                                                       : __builtin_amdgcn_exp2f(m_old * c - msc);
      m_run[qb] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], c, -msc));
          if (masked) e = (s[kb][qb][r] == -__builtin_inff()) ? 0.f : e;
          pv[r] = e;
          rs += e;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int b = half * 8;
          pb[kb * 2 + half][qb] =
              u32x4_t{E::pack(pv[b + 0], pv[b + 1]), E::pack(pv[b + 2], pv[b + 3]),
                      E::pack(pv[b + 4], pv[b + 5]), E::pack(pv[b + 6], pv[b + 7])};
        }
      }
      l_part[qb] = l_part[qb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned char* vrow = vts + vrow_off[db];
#pragma unroll
      for (int ks2 = 0; ks2 < BC / 16; ++ks2) {
        const int unit = (ks2 * 2 + hh) ^ vswz[db];
        const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(vrow + unit * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = E::mfma(vf, pb[ks2][qb], oacc[db][qb]);
      }
    }
  };

  // ---- main loop over key tiles (double-buffered LDS, one barrier per tile) --------
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < n_kt;
    if (more) load_tile(j + 1);
    if (wave_live && j < w_kt) compute_tile(buf, j);
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O~ / l, L = m*scale + ln(l) -----------------------------------
  if (!wave_live) return;
  const float kLn2 = 0.69314718055994530942f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_part[qb] + __shfl_xor(l_part[qb], 32);
    const int qi = wq0 + qb * 32 + l32;
    if (qi >= N) continue;
    const float inv = 1.0f / l_tot;
    uint16_t* orow = p.o + head + (size_t)qi * dstride;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dcol = db * 32 + g * 8 + hh * 4;
        const f32x16_t& a = oacc[db][qb];
        const uint32_t w0 = E::pack(a[4 * g + 0] * inv, a[4 * g + 1] * inv);
        const uint32_t w1 = E::pack(a[4 * g + 2] * inv, a[4 * g + 3] * inv);
        if (EXACT_D) {
          *reinterpret_cast<u32x2_t*>(orow + dcol) = u32x2_t{w0, w1};
        } else {
          const uint16_t h4[4] = {(uint16_t)(w0 & 0xffffu), (uint16_t)(w0 >> 16),
                                  (uint16_t)(w1 & 0xffffu), (uint16_t)(w1 >> 16)};
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (dcol + t < p.d) orow[dcol + t] = h4[t];
        }
      }
    if (hh == 0) {
      const float msc = m_run[qb] * c;
      p.lse[(size_t)bh * N + qi] = (msc + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

}  // namespace fa
