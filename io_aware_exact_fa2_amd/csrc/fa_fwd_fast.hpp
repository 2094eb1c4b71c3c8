// fa_fwd_fast.hpp — FA2-order attention forward for gfx950 (MI355X), fast path for
// head dims 64 and 128.
//
// Algorithm ([P1] currybab.bearblog.dev, "Triton으로 FlashAttention 구현하기 전에 -
// FA1, 2 forward pass", section "FlashAttention 2 forward pass 알고리즘 분석"): the
// query row block is the outer loop (one workgroup per query block, head and batch:
// the section's sequence parallelism), key/value blocks stream through LDS in the
// inner loop, each row keeps its running max and sum on chip, rescales the
// unnormalised output by alpha = exp(m_old - m_new) only, and divides once at the
// end (the section's per-block update and epilogue equations). Waves own disjoint
// query rows (split-Q), so no cross-wave merge exists.
//
// gfx950 mapping (differences from the generic kernel in fa_fwd_generic.hpp):
//   * K and V tiles are copied HBM -> LDS by global_load_lds_dwordx4 (no register
//     staging, no VALU work), one tile ahead, into two LDS stages; one barrier per
//     tile. Both stay row-major in LDS; K rows carry one 16-byte pad chunk and V rows
//     four, which makes every LDS read below bank-conflict free with compile-time
//     address offsets (the pad slots are simply not written).
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}: each lane owns
//     one query column, so the running max/sum and the alpha rescale are in-lane and
//     the S^T accumulator, rounded to 16 bits, is the B operand of the P V MFMA.
//     Key rows enter the S^T MFMA with bits 2 and 3 of the row index swapped so a
//     lane's 8 values of one 16-key step are 8 consecutive keys.
//   * The V^T operand is read with ds_read_b64_tr_b16: in each 16-lane group, lane i
//     receives column i of the 4 rows the group loads, i.e. 4 consecutive keys of
//     one head-dim column; two such reads form one 8-key MFMA operand.
//   * The two wave halves holding the same query exchange the row max with one
//     v_permlane32_swap; the row sum is accumulated per lane in fp32 and combined
//     once at the end.
//   * exp2 with the log2(e) factor folded into the scale: p = exp2(s*c - m*c), one
//     FMA and one v_exp_f32 per score; the max is tracked in those log2 units.
//   * Optional lazy rescale (TAU > 0): the reference max of a row is raised (and O~,
//     l rescaled by alpha) only when a tile's max exceeds it by more than TAU in
//     log2 units; otherwise the old reference is kept, so probabilities stay below
//     2^TAU. Softmax is invariant to the reference, so O and L are unchanged; TAU = 0
//     is the literal update of every tile, with the multiply skipped when no row of
//     the wave changed its max (alpha = 1).
//   * Causal: key tiles past the workgroup's last query are never loaded, a wave
//     skips tiles past its own last query, and element masks are applied only on
//     diagonal and ragged-tail tiles ([P2] iq-universe.github.io, "FlashAttention은
//     어떻게 O(N²) 메모리 벽을 넘었나", section "v2와 v3": blocks above the diagonal
//     are skipped whole).
#pragma once

#include "fa_common.hpp"

namespace fa {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

template <int D_, int QB_, int NW_, int BC_>
struct FastGeom {
  static constexpr int D = D_;
  static constexpr int QB = QB_;
  static constexpr int NW = NW_;
  static constexpr int BC = BC_;
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * QB * 32;
  static constexpr int CPR = D / 8;              // 16-byte chunks of data per row
  static constexpr int KPC = CPR + 1;            // K row pitch in LDS chunks
  static constexpr int VPC = CPR + 4;            // V row pitch in LDS chunks
  static constexpr int K_CHUNKS = BC * KPC;
  static constexpr int V_CHUNKS = BC * VPC;
  static constexpr int K_INSTR = K_CHUNKS / 64;  // 1 KB wave instructions per tile
  static constexpr int V_INSTR = V_CHUNKS / 64;
  static constexpr int K_PER_WAVE = (K_INSTR + NW - 1) / NW;
  static constexpr int V_PER_WAVE = (V_INSTR + NW - 1) / NW;
  static constexpr int LDS = 2 * 16 * (K_CHUNKS + V_CHUNKS);
  static_assert(D == 64 || D == 128, "fast path head dims");
  static_assert(BC % 64 == 0, "tile loads are whole wave instructions");
  static_assert(K_CHUNKS % 64 == 0 && V_CHUNKS % 64 == 0, "tile loads are whole wave instructions");
};

template <bool BF16, int D, bool CAUSAL, int QB, int NW, int BC, int TAU, int WPE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
fa_fwd_fast_kernel(const Params p) {
  using G = FastGeom<D, QB, NW, BC>;
  using E = Elt<BF16>;
  __shared__ u32x4_t ks0[G::K_CHUNKS];
  __shared__ u32x4_t vs0[G::V_CHUNKS];
  __shared__ u32x4_t ks1[G::K_CHUNKS];
  __shared__ u32x4_t vs1[G::V_CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int N = p.N;

  int bh, qt;
  decode_tile<CAUSAL>(p, blockIdx.x, bh, qt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ qg = p.q + head;
  const uint16_t* __restrict__ kg = p.k + head;
  const uint16_t* __restrict__ vg = p.v + head;

  const int q0 = qt * G::BR;
  const int wq0 = q0 + wid * QB * 32;
  const int q_end = min(q0 + G::BR, N);
  const int n_kt = CAUSAL ? (q_end + BC - 1) / BC : (N + BC - 1) / BC;
  const bool wave_live = wq0 < N;
  const int w_last_q = min(wq0 + QB * 32, N) - 1;
  const int w_kt = CAUSAL ? min(n_kt, w_last_q / BC + 1) : n_kt;

  // ---- per-lane element offsets (within a tile) of the chunks this wave copies ----
  int koff[G::K_PER_WAVE], voff[G::V_PER_WAVE];
#pragma unroll
  for (int ii = 0; ii < G::K_PER_WAVE; ++ii) {
    const int i = wid + ii * NW;
    const int f = i * 64 + lane, row = f / G::KPC, ch = f % G::KPC;
    koff[ii] = (i < G::K_INSTR && ch < G::CPR) ? row * D + ch * 8 : -1;
  }
#pragma unroll
  for (int ii = 0; ii < G::V_PER_WAVE; ++ii) {
    const int i = wid + ii * NW;
    const int f = i * 64 + lane, row = f / G::VPC, ch = f % G::VPC;
    voff[ii] = (i < G::V_INSTR && ch < G::CPR) ? row * D + ch * 8 : -1;
  }

  // HBM -> LDS copy of key/value tile j into one stage. Rows past N are clamped to
  // row N-1 (always a valid address); their scores are masked to -inf, so their
  // probabilities are exactly 0 and the duplicated values contribute nothing.
  auto issue_tile = [&](u32x4_t* kst, u32x4_t* vst, int j) {
    const int k0 = j * BC;
    const bool tail = k0 + BC > N;
    const uint16_t* kt = kg + (size_t)k0 * D;
    const uint16_t* vt = vg + (size_t)k0 * D;
#pragma unroll
    for (int ii = 0; ii < G::K_PER_WAVE; ++ii) {
      const int i = wid + ii * NW;
      if (i < G::K_INSTR) {
        int off = koff[ii];
        if (tail && off >= 0 && k0 + off / D >= N) off = (N - 1 - k0) * D + (off & (D - 1));
        if (off >= 0)
          __builtin_amdgcn_global_load_lds(kt + off, (lds_void_t*)(kst + i * 64), 16, 0, 0);
      }
    }
#pragma unroll
    for (int ii = 0; ii < G::V_PER_WAVE; ++ii) {
      const int i = wid + ii * NW;
      if (i < G::V_INSTR) {
        int off = voff[ii];
        if (tail && off >= 0 && k0 + off / D >= N) off = (N - 1 - k0) * D + (off & (D - 1));
        if (off >= 0)
          __builtin_amdgcn_global_load_lds(vt + off, (lds_void_t*)(vst + i * 64), 16, 0, 0);
      }
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T), in registers for the whole loop ------
  u32x4_t qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = wq0 + qb * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (qi < N) x = ld16(qg + (size_t)qi * D + ds * 16 + hh * 8);
      qf[qb][ds] = x ^ p.qsign;
    }
  }

  // ---- running state ---------------------------------------------------------------
  f32x16_t oacc[D / 32][QB];
  float ms[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    ms[qb] = 0.f;
    l_part[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  }
  const float c = p.c;
  // lane-constant LDS byte offsets of the K operand row and the V^T transposed reads
  const int k_lane = (key_of_row(l32) * G::KPC + hh) * 16;
  const int g16 = lane >> 4, t4 = (lane & 15) >> 2, u4 = lane & 3;
  const int v_lane = (((g16 >> 1) * 8 + t4) * G::VPC + (g16 & 1) * 2 + (u4 >> 1)) * 16 + (u4 & 1) * 8;

  auto compute_tile = [&](const u32x4_t* kst, const u32x4_t* vst, int j) {
    const int k0 = j * BC;
    const unsigned char* kbase = reinterpret_cast<const unsigned char*>(kst) + k_lane;
    const unsigned char* vbase = reinterpret_cast<const unsigned char*>(vst) + v_lane;

    // S^T = K Q^T (raw dot products)
    f32x16_t s[BC / 32][QB];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const u32x4_t kf =
            *reinterpret_cast<const u32x4_t*>(kbase + (kb * 32 * G::KPC + 2 * ds) * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = E::mfma(kf, qf[qb][ds], s[kb][qb]);
      }
    }

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
            if (key >= N || (CAUSAL && key > qi)) s[kb][qb][r] = -__builtin_inff();
          }
      }
    }

    // online softmax: one query per lane pair (lane, lane^32)
    u32x4_t pb[BC / 16][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][qb][r]);
      const float mxs = xhalf_max(mx) * c;
      if (j == 0) {
        ms[qb] = mxs;  // tile 0 holds key 0, allowed for every row: mxs is finite
      } else {
        const bool grow = mxs > ms[qb] + (float)TAU;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float ms_new = __builtin_fmaxf(ms[qb], mxs);
          const float alpha = __builtin_amdgcn_exp2f(ms[qb] - ms_new);
          ms[qb] = ms_new;
          l_part[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
        }
      }
      const float msc = ms[qb];
      // row sum in fp32 of the unrounded probabilities (two chains for latency)
      float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // c > 0 on this path, so a masked score (-inf) gives exp2(-inf) = 0 exactly
          pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], c, -msc));
          if (r & 1) lsum1 += pv[r];
          else lsum0 += pv[r];
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int b = half * 8;
          pb[kb * 2 + half][qb] =
              u32x4_t{E::pack(pv[b + 0], pv[b + 1]), E::pack(pv[b + 2], pv[b + 3]),
                      E::pack(pv[b + 4], pv[b + 5]), E::pack(pv[b + 6], pv[b + 7])};
        }
      }
      const float lsum = l_part[qb] + (lsum0 + lsum1);
      l_part[qb] = lsum;
    }

    // O^T += V^T P^T: V^T fragments straight from row-major V by transposed reads
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int st = 0; st < BC / 16; ++st) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(vbase + ((16 * st + 0) * G::VPC + 4 * db) * 16));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(vbase + ((16 * st + 4) * G::VPC + 4 * db) * 16));
        const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t vf = {lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = E::mfma(vf, pb[st][qb], oacc[db][qb]);
      }
    }
  };

  // ---- main loop: stage 0 holds even tiles, stage 1 odd tiles ------------------------
  issue_tile(ks0, vs0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int j = 0; j < n_kt; j += 2) {
    if (j + 1 < n_kt) issue_tile(ks1, vs1, j + 1);
    if (wave_live && j < w_kt) compute_tile(ks0, vs0, j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 >= n_kt) break;
    if (j + 2 < n_kt) issue_tile(ks0, vs0, j + 2);
    if (wave_live && j + 1 < w_kt) compute_tile(ks1, vs1, j + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: O = O~ / l, L = (m*c + log2 l) * ln 2 ------------------------------
  if (!wave_live) return;
  const float kLn2 = 0.69314718055994530942f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = xhalf_sum(l_part[qb]);
    const int qi = wq0 + qb * 32 + l32;
    if (qi >= N) continue;
    const float inv = 1.0f / l_tot;
    uint16_t* orow = p.o + head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dcol = db * 32 + g * 8 + hh * 4;
        const f32x16_t& a = oacc[db][qb];
        const uint32_t w0 = E::pack(a[4 * g + 0] * inv, a[4 * g + 1] * inv);
        const uint32_t w1 = E::pack(a[4 * g + 2] * inv, a[4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + dcol) = u32x2_t{w0, w1};
      }
    if (hh == 0) p.lse[(size_t)bh * N + qi] = (ms[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
}

}  // namespace fa
