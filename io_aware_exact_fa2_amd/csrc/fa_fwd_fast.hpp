// fa_fwd_fast.hpp — FA2-order attention forward for gfx950 (MI355X), 32 queries per wave:
// the fast path for head dim 64 (the template also builds at 128, which the library
// serves with the wide kernel).
//
// Algorithm ([P1] currybab.bearblog.dev, "Triton으로 FlashAttention 구현하기 전에 -
// FA1, 2 forward pass", section "FlashAttention 2 forward pass 알고리즘 분석"): the
// query row block is the outer loop (one workgroup per query block, head and batch:
// the section's sequence parallelism), key/value blocks stream through LDS in the
// inner loop, each row keeps its running max and sum on chip, rescales the
// unnormalised output by alpha = exp(m_old - m_new) only, and divides once at the
// end (the section's per-block update and epilogue equations). Waves own disjoint
// query rows (split-Q), so no cross-wave merge exists. With SPLIT, workgroup (s, head,
// query block) covers only the keys of split s and writes its normalized partial O and
// partial L in float32 for the split-KV merge (fa_fwd_split.hpp).
//
// gfx950 mapping:
//   * K and V tiles are copied HBM -> LDS by buffer_load_dwordx4 ... lds (no register
//     staging, no VALU work) into two LDS slots each; one barrier per tile. Each tile
//     is a whole number of 1 KB wave copies and every wave issues the same number,
//     with no branches (past the last tile a wave re-copies the last tile into a
//     slot that is already free), so the copies can be scheduled between MFMAs.
//   * K runs one tile ahead of V: while tile j is finished, the S^T MFMAs of tile
//     j+1 are interleaved with the exponentials of tile j, and the P V MFMAs of tile
//     j with the row max of tile j+1, so the matrix cores and the VALU work on
//     different tiles at the same time (the order is imposed on the machine
//     scheduler with sched_group_barrier patterns).
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}: each lane owns
//     one query column, so the running max/sum and the alpha rescale are in-lane and
//     the S^T accumulator, rounded to 16 bits, is the B operand of the P V MFMA.
//     Key rows enter the S^T MFMA with bits 2 and 3 of the row index swapped so a
//     lane's 8 values of one 16-key step are 8 consecutive keys.
//   * K and V stay row-major in LDS, with the 16-byte chunks of each row XOR-
//     swizzled by the row index so every ds_read_b128 of K and every
//     ds_read_b64_tr_b16 of V is bank-conflict free; the per-lane addresses are
//     computed once, the per-step offsets are compile-time.
//   * The V^T operand is read with ds_read_b64_tr_b16: in each 16-lane group, lane i
//     receives column i of the 4 rows the group loads, i.e. 4 consecutive keys of
//     one head-dim column; two such reads form one 8-key MFMA operand.
//   * The two wave halves holding the same query exchange the row max with one
//     v_permlane32_swap; the row sum is accumulated per lane in fp32 and combined
//     once at the end.
//   * exp2 with the log2(e) factor folded into the scale: p = exp2(s*c - m*c), one
//     FMA and one v_exp_f32 per score; the max is tracked in those log2 units.
//   * Lazy rescale (tau > 0, a kernel argument): the reference max of a row is raised
//     (and O~, l rescaled by alpha) only when a tile's max exceeds it by more than tau
//     in log2 units; otherwise the old reference is kept, so probabilities stay below
//     2^tau. Softmax is invariant to the reference, so O and L are unchanged; tau = 0
//     is the literal update of every tile, with the multiply skipped when no row of
//     the wave changed its max (alpha = 1).
//   * Causal: key tiles past the workgroup's last query are never computed, a wave
//     skips tiles past its own last query, and element masks are applied only on
//     diagonal and ragged-tail tiles ([P2] iq-universe.github.io, "FlashAttention은
//     어떻게 O(N²) 메모리 벽을 넘었나", section "v2와 v3": blocks above the diagonal
//     are skipped whole).
#pragma once

#include "fa_common.hpp"

// Interleave patterns (instructions per pipeline step) given to the machine scheduler.
#ifndef FA_SG_B_VALU
#define FA_SG_B_VALU 6    // VALU per S^T MFMA step (exponentials of the previous tile)
#endif
#ifndef FA_SG_C_VALU
#define FA_SG_C_VALU 2    // VALU per P V MFMA step (row max of the next tile)
#endif
#ifndef FA_SG_PREFETCH
#define FA_SG_PREFETCH 5  // MFMA steps an LDS operand read runs ahead (2: 2.4% slower at d = 64)
#endif
#ifndef FA_SG_ON
#define FA_SG_ON 1
#endif

namespace fa {

template <int D_, int NW_, int BC_, int QB_ = 1>
struct FastGeom {
  static constexpr int D = D_;
  static constexpr int NW = NW_;
  static constexpr int BC = BC_;
  static constexpr int QB = QB_;                 // 32-query blocks per wave
  static constexpr int BR = NW * 32 * QB;        // queries per workgroup
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int CHUNKS = BC * CPR;        // chunks per K (or V) tile
  static constexpr int INSTR = CHUNKS / 64;      // 1 KB wave copies per tile and tensor
  static constexpr int PER_WAVE = INSTR / NW;    // copies per wave per tile and tensor
  static constexpr int NQK = (BC / 32) * (D / 16);  // S^T MFMA steps per tile
  static constexpr int NPV = (D / 32) * (BC / 16);  // P V MFMA steps per tile
  static_assert(D == 64 || D == 128, "fast path head dims");
  static_assert(BC % 32 == 0 && CHUNKS % 64 == 0, "whole MFMA blocks and wave copies");
  static_assert(INSTR % NW == 0 && PER_WAVE >= 1, "every wave issues the same copies");
  static_assert(2 * PER_WAVE <= NQK, "copies fit in the S^T pipeline steps");
  static_assert(QB == 1 || QB == 2, "one or two query blocks per wave");
};

template <bool BF16, int D, bool CAUSAL, int NW, int BC, int WPE, bool SPLIT = false, int QB = 1>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
fa_fwd_fast_kernel(const Params p) {
  using G = FastGeom<D, NW, BC, QB>;
  using E = Elt<BF16>;
  constexpr int CPR = G::CPR, NQK = G::NQK, NPV = G::NPV;
  constexpr int NSC = QB * (BC / 2);   // scores per lane and tile
  constexpr int SPS = NSC / NQK;       // scores exponentiated per S^T step
  constexpr int MPS = NSC / NPV;       // scores max-reduced per P V step
  constexpr int SGP = FA_SG_PREFETCH;
  static_assert(SPS % 2 == 0 && MPS >= 1, "pipeline step split");
  __shared__ u32x4_t ks0[G::CHUNKS];
  __shared__ u32x4_t vs0[G::CHUNKS];
  __shared__ u32x4_t ks1[G::CHUNKS];
  __shared__ u32x4_t vs1[G::CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int N = p.N;

  int bh, qt, split = 0;
  if constexpr (SPLIT) {
    // split-major grid: every split sees the same (head, tile) decode
    const int per = p.n_qt * p.BH;
    split = blockIdx.x / per;
    decode_tile<CAUSAL>(p, blockIdx.x % per, bh, qt);
  } else {
    decode_tile<CAUSAL>(p, blockIdx.x, bh, qt);
  }
  // keys [kofs, kofs + Nk) of the head; key indices below are relative to kofs (the
  // whole head unless this is a split-KV partial pass)
  const int kofs = SPLIT ? split * p.split_keys : 0;
  const int Nk = SPLIT ? min(N - kofs, p.split_keys) : N;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ qg = p.q + head;
  const uint16_t* __restrict__ kg = p.k + head + (size_t)kofs * D;
  const uint16_t* __restrict__ vg = p.v + head + (size_t)kofs * D;

  static_assert(!(SPLIT && QB == 2), "the split-KV pass runs one query block per wave");
  const int q0 = qt * G::BR;
  // wave w owns the 32-query block w, and with two blocks per wave also block
  // 2 NW - 1 - w (under the causal mask the two blocks' work then differs by the same
  // amount in every wave)
  int qbase[QB];
  qbase[0] = q0 + wid * 32;
  if constexpr (QB == 2) qbase[QB - 1] = q0 + 32 * (2 * NW - 1 - wid);
  const int wq0 = qbase[0];  // the wave's first query
  const int q_end = min(q0 + G::BR, N);
  const int n_kt = CAUSAL ? (min(q_end - kofs, Nk) + BC - 1) / BC : (Nk + BC - 1) / BC;
  const bool wave_live = wq0 < N;
  const int w_last_q = min(qbase[QB - 1] + 32, N) - 1;
  const int w_kt = CAUSAL ? min(n_kt, (w_last_q - kofs) / BC + 1) : n_kt;
  if constexpr (SPLIT) {
    // Splits start at multiples of the query tile, so under the causal mask a split
    // either starts at or before q0 (every query of the tile sees its first key) or
    // after the tile's last query (empty: partial L = -inf, partial O = 0).
    if (n_kt <= 0) {
      const int qi = q0 + tid;
      if (tid < G::BR && qi < N) {
        const size_t row = ((size_t)split * p.BH + bh) * N + qi;
        p.l_part[row] = -__builtin_inff();
        float* orow = p.o_part + row * D;
        for (int c4 = 0; c4 < D; c4 += 4)
          *reinterpret_cast<float4*>(orow + c4) = float4{0.f, 0.f, 0.f, 0.f};
      }
      return;
    }
  }

  // ---- HBM -> LDS copies ---------------------------------------------------------
  // Lane `lane` of copy instruction i writes LDS chunk 64 i + lane = (row, physical
  // chunk); it fetches the logical chunk that the swizzle puts there. Element
  // offsets within a tile are computed once.
  int koff[G::PER_WAVE], voff[G::PER_WAVE];
#pragma unroll
  for (int ii = 0; ii < G::PER_WAVE; ++ii) {
    const int f = (wid + ii * NW) * 64 + lane, row = f / CPR, ph = f % CPR;
    koff[ii] = row * D + (ph ^ swz_k<D>(row)) * 8;
    voff[ii] = row * D + (ph ^ swz_v<D>(row)) * 8;
  }
  // One copy of tile j, as a buffer load with an LDS destination. The buffer resource
  // spans the tile's rows below N, so chunks of rows past N read as zeros (their
  // scores are masked to -inf, so they contribute exactly 0). A copy past the last
  // tile re-fetches the last tile into a slot nobody reads. The buffer form is used
  // (rather than global_load_lds) because its completion is tracked by vmcnt alone,
  // so the LDS operand reads of the pipeline keep partial lgkmcnt waits.
  auto copy = [&](const uint16_t* src, u32x4_t* dst, int off, int ii, int j) {
    const int k0 = min(j, n_kt - 1) * BC;
    const int bytes = min(Nk - k0, BC) * D * 2;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src + (size_t)k0 * D), (short)0, bytes, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + (wid + ii * NW) * 64), 16,
                                             off * 2, 0, 0, 0);
  };
  struct Copies {
    u32x4_t* k_dst;
    u32x4_t* v_dst;
    int jk, jv;
  };
  constexpr int NDMA = 2 * G::PER_WAVE;
  auto copy_step = [&](const Copies& cp, int i) {
    if (i < G::PER_WAVE) copy(kg, cp.k_dst, koff[i], i, cp.jk);
    else if (i < NDMA) copy(vg, cp.v_dst, voff[i - G::PER_WAVE], i - G::PER_WAVE, cp.jv);
  };
  auto copy_all = [&](const Copies& cp) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) copy_step(cp, i);
  };

  // ---- Q fragments (B operand of S^T = K Q^T), in registers for the whole loop ------
  u32x4_t qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qbase[qb] + l32;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (qi < N) x = ld16(qg + (size_t)qi * D + ds * 16 + hh * 8);
      qf[qb][ds] = x ^ p.qsign;
    }
  }

  // ---- running state ---------------------------------------------------------------
  f32x16_t oacc[QB][D / 32];
  float ms[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
    ms[qb] = 0.f;
    l_part[qb] = 0.f;
  }
  const float c = p.c;

  // ---- per-lane LDS read addresses ---------------------------------------------------
  // K operand of step (kb, ds): row 32 kb + rho(l32), logical chunk 2 ds + hh. The
  // swizzle of that row does not depend on kb, so one address per ds (kb adds a
  // compile-time offset). Bank check: the 16 lanes of a b128 quarter-wave read 16
  // different rows at one logical chunk; the row-dependent XOR sends them to 16
  // different bank quads.
  int kaddr[D / 16];
  {
    const int row = key_of_row(l32);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      kaddr[ds] = (row * CPR + ((2 * ds + hh) ^ swz_k<D>(row))) * 16;
  }
  // V^T operand of step (db, st), half r: lane (group g16, t4, u4) reads 8 bytes of
  // row 16 st + 8 (g16 >> 1) + 4 r + t4 at column 32 db + 16 (g16 & 1) + 4 u4. The
  // swizzle depends on the row only through t4, so one address per db. Bank check:
  // the 32 lanes of a half-wave read 4 rows x 4 chunks; the XOR by 4*(row & 3)
  // (d = 128) or 4*((row >> 1) & 1) (d = 64) spreads them over distinct banks.
  int vaddr[D / 32];
  {
    const int g16 = lane >> 4, t4 = (lane & 15) >> 2, u4 = lane & 3;
    const int row = (g16 >> 1) * 8 + t4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vaddr[db] = (row * CPR + ((4 * db + 2 * (g16 & 1) + (u4 >> 1)) ^ swz_v<D>(row))) * 16 +
                  (u4 & 1) * 8;
  }
  auto k_frag = [&](const u32x4_t* kst, int i) {
    const int kb = i % (BC / 32), ds = i / (BC / 32);
    return *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const unsigned char*>(kst) +
                                             kaddr[ds] + kb * 32 * CPR * 16);
  };
  auto v_frag = [&](const u32x4_t* vst, int i) {
    const int db = i % (D / 32), st = i / (D / 32);
    const unsigned char* b = reinterpret_cast<const unsigned char*>(vst) + vaddr[db];
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(b + (16 * st + 0) * CPR * 16));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(b + (16 * st + 4) * CPR * 16));
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };

  typedef f32x16_t STile[BC / 32][QB];  // S^T accumulators of one key tile
  // score e of a tile: query block e / (BC / 2); within it, f = e % (BC / 2) is key
  // block f / 16, accumulator register f % 16
  auto zero = [](STile& s) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
  };

  // -inf on keys past N and, under the causal mask, on keys after the query; only
  // tiles that reach past N or cross the diagonal need it
  auto mask = [&](STile& s, int j) {
    const int k0 = j * BC;
    const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > wq0 - kofs);
    if (!masked) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = qbase[qb] + l32 - kofs;  // the query, in key coordinates
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + key_of_reg(r, hh);
          if (key >= Nk || (CAUSAL && key > qi)) s[kb][qb][r] = -__builtin_inff();
        }
    }
  };

  // m_new = max(m_old, rowmax S); alpha = exp2(m_old - m_new) rescales l and O~. The
  // whole wave skips it when no row needs it (alpha = 1), or, with tau > 0, when no
  // row's max rose by more than tau (log2 units).
  auto grow_max = [&](int qb, float mxs) {
    if (__builtin_amdgcn_ballot_w64(mxs > ms[qb] + p.tau) != 0) {
      const float ms_new = __builtin_fmaxf(ms[qb], mxs);
      const float alpha = __builtin_amdgcn_exp2f(ms[qb] - ms_new);
      ms[qb] = ms_new;
      l_part[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
    }
  };

  u32x4_t pb[QB][BC / 16];  // P~ of the current tile, packed as P V operands

  // Block B: S^T of tile j+1 (MFMA) interleaved with the exponentials of tile j (VALU)
  // and this wave's copies of the following tiles (VMEM). Each K operand read from LDS
  // feeds one MFMA per query block.
  auto qk_exp = [&](const u32x4_t* k_next, STile& s_next, const STile& s_cur,
                    const Copies& cp) {
    zero(s_next);
    float msc[QB], lsum[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      msc[qb] = ms[qb];
      lsum[qb][0] = 0.f;
      lsum[qb][1] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int kb = i % (BC / 32), ds = i / (BC / 32);
      const u32x4_t kf = k_frag(k_next, i);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s_next[kb][qb] = E::mfma(kf, qf[qb][ds], s_next[kb][qb]);
#pragma unroll
      for (int e = i * SPS; e < (i + 1) * SPS; e += 2) {
        const int qb = e / (BC / 2), f = e % (BC / 2);
        // c > 0 on this path, so a masked score (-inf) gives exp2(-inf) = 0 exactly
        const float p0 =
            __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[f / 16][qb][f % 16], c, -msc[qb]));
        const float p1 =
            __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[f / 16][qb][(f + 1) % 16], c, -msc[qb]));
        const uint32_t w = E::pack(p0, p1);
        pb[qb][f / 8][(f % 8) / 2] = w;
        if constexpr (BF16) {
          lsum[qb][0] += p0;
          lsum[qb][1] += p1;
        } else {
          // half-precision P: l sums the rounded pair (one dot2), each term within 2^-11
          // of its probability, so L moves by at most that relative amount
          float& acc = lsum[qb][(f / 2) % 2];
          acc = E::sum2(w, acc);
        }
      }
      copy_step(cp, i);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_part[qb] += lsum[qb][0] + lsum[qb][1];
    // keep the exponentials in this block (no sinking into the P V block): a use of the
    // packed operands here. (A tied in/out operand did the same but cost 8 register
    // moves per tile to bring them back into the operand registers.)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int st = 0; st < BC / 16; ++st) asm volatile("" ::"v"(pb[qb][st]));
#if FA_SG_ON
    __builtin_amdgcn_sched_group_barrier(0x100, SGP, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, FA_SG_B_VALU, 0);
      }
      if (i < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (i + SGP < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#endif
  };

  // Block C: P V of tile j (MFMA) interleaved with the row max of tile j+1 (VALU); each
  // V^T operand read feeds one MFMA per query block. mx: the lane's max per query block.
  auto pv_max = [&](const u32x4_t* v_cur, const STile& s_next, float (&mx)[QB]) {
    float m[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m[qb][0] = m[qb][1] = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int db = i % (D / 32), st = i / (D / 32);
      const u32x4_t vf = v_frag(v_cur, i);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma(vf, pb[qb][st], oacc[qb][db]);
#pragma unroll
      for (int e = i * MPS; e < (i + 1) * MPS; ++e) {
        const int qb = e / (BC / 2), f = e % (BC / 2);
        m[qb][e & 1] = __builtin_fmaxf(m[qb][e & 1], s_next[f / 16][qb][f % 16]);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float x = __builtin_fmaxf(m[qb][0], m[qb][1]);
      asm volatile("" : "+v"(x));
      mx[qb] = x;
    }
#if FA_SG_ON
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * SGP, 1);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, FA_SG_C_VALU, 1);
      }
      if (i + SGP < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
#endif
  };

  // One key tile j whose masked S^T is in s_cur and whose max is already folded into
  // ms: exponentials and P V of tile j, overlapped with the S^T, mask and max of tile
  // j+1 (from K slot k_next). On a wave's last tile the look-ahead reads a stale but
  // valid K slot and its result is dropped (`next` false: no max update).
  auto tile = [&](const STile& s_cur, STile& s_next, const u32x4_t* k_next,
                  const u32x4_t* v_cur, int j, bool next, const Copies& cp) {
    qk_exp(k_next, s_next, s_cur, cp);
    mask(s_next, j + 1);
    float mx[QB];
    pv_max(v_cur, s_next, mx);
    if (next) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) grow_max(qb, xhalf_max(mx[qb]) * c);
    }
  };

  // ---- main loop ---------------------------------------------------------------------
  // Slots: K tile t lives in ks[t % 2], V tile t in vs[t % 2]. While tile j is being
  // finished (V_j in vs[j%2]) the S^T of tile j+1 is computed from ks[(j+1)%2], and
  // the copies of K_{j+2} (into ks[j%2]) and V_{j+1} (into vs[(j+1)%2]) are in flight.
  STile sa, sb;
  {
    const Copies c0 = {ks0, vs0, 0, 0};
    copy_all(c0);
#pragma unroll
    for (int ii = 0; ii < G::PER_WAVE; ++ii) copy(kg, ks1, koff[ii], ii, 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wave_live) {
    zero(sa);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int kb = i % (BC / 32), ds = i / (BC / 32);
      const u32x4_t kf = k_frag(ks0, i);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sa[kb][qb] = E::mfma(kf, qf[qb][ds], sa[kb][qb]);
    }
    mask(sa, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sa[kb][qb][r]);
      ms[qb] = xhalf_max(mx) * c;  // tile 0 holds key 0, allowed for every row: finite
    }
  }
  __syncthreads();  // every wave is done with ks0 before K_2 overwrites it
  for (int j = 0; j < n_kt; j += 2) {
    const Copies ce = {ks0, vs1, j + 2, j + 1};
    if (wave_live && j < w_kt) tile(sa, sb, ks1, vs0, j, j + 1 < w_kt, ce);
    else copy_all(ce);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 >= n_kt) break;
    const Copies co = {ks1, vs0, j + 3, j + 2};
    if (wave_live && j + 1 < w_kt) tile(sb, sa, ks0, vs1, j + 1, j + 2 < w_kt, co);
    else copy_all(co);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: O = O~ / l, L = (m*c + log2 l) * ln 2 ------------------------------
  if (!wave_live) return;
  const float kLn2 = 0.69314718055994530942f;
  if constexpr (QB == 1) {
    const float l_tot = xhalf_sum(l_part[0]);
    const int qi = wq0 + l32;  // rows past N (finite, from clamped or zero rows) are never stored
    const float inv = 1.0f / l_tot;
    if constexpr (SPLIT) {
      if (qi >= N) return;
      const size_t row = ((size_t)split * p.BH + bh) * N + qi;
      float* prow = p.o_part + row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& a = oacc[0][db];
          *reinterpret_cast<float4*>(prow + db * 32 + g * 8 + hh * 4) =
              float4{a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv};
        }
      if (hh == 0) p.l_part[row] = (ms[0] + __builtin_amdgcn_logf(l_tot)) * kLn2;
      return;
    }
    // O leaves through LDS (the loop ended at a barrier after every copy landed, so the K
    // and V slots are idle): the wave writes its 32 rows into its own part of them (a lane
    // holds 8 bytes of one row per write) and stores 16-byte chunks of whole rows, instead
    // of 8-byte pieces over 32 rows per store instruction, in the o_pos / o_swap layout.
    static_assert(NW <= 4 && 2 * 32 * CPR <= G::CHUNKS, "two waves' O tiles fit one slot");
    unsigned char* ot =
        reinterpret_cast<unsigned char*>((wid < 2 ? ks0 : vs0) + (wid & 1) * 32 * CPR);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16_t& a = oacc[0][db];
        const uint32_t w0 = E::pack(a[4 * g + 0] * inv, a[4 * g + 1] * inv);
        const uint32_t w1 = E::pack(a[4 * g + 2] * inv, a[4 * g + 3] * inv);
        const int c = db * 4 + g;  // 16-byte chunk of row l32; this lane holds half hh
        *reinterpret_cast<u32x2_t*>(ot + o_half_off<CPR>(l32, c, hh)) = u32x2_t{w0, w1};
      }
    if (hh == 0 && qi < N)
      p.lse[(size_t)bh * N + qi] = (ms[0] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own writes, in order
#pragma unroll
    for (int it = 0; it < CPR / 2; ++it) {
      const int rr = (64 / CPR) * it + lane / CPR, c = lane % CPR;
      const u32x4_t x = o_chunk_read<CPR>(ot, rr, c);
      if (wq0 + rr < N)
        *reinterpret_cast<u32x4_t*>(p.o + head + (size_t)(wq0 + rr) * D + c * 8) = x;
    }
  } else {
    // Two query blocks: the wave's 64 rows go through a staging area of their own (the
    // key/value slots are too small for them), 16-byte chunks of whole rows per store,
    // in the o_pos / o_swap layout; row 32 qb + r of the area is query qbase[qb] + r.
    __shared__ __attribute__((aligned(16))) u32x4_t ostage[NW * 64 * CPR];
    unsigned char* ot = reinterpret_cast<unsigned char*>(ostage + wid * 64 * CPR);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = xhalf_sum(l_part[qb]);
      const float inv = 1.0f / l_tot;
      const int rr = 32 * qb + l32;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& a = oacc[qb][db];
          const uint32_t w0 = E::pack(a[4 * g + 0] * inv, a[4 * g + 1] * inv);
          const uint32_t w1 = E::pack(a[4 * g + 2] * inv, a[4 * g + 3] * inv);
          *reinterpret_cast<u32x2_t*>(ot + o_half_off<CPR>(rr, db * 4 + g, hh)) = u32x2_t{w0, w1};
        }
      const int qi = qbase[qb] + l32;
      if (hh == 0 && qi < N)
        p.lse[(size_t)bh * N + qi] = (ms[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own writes, in order
#pragma unroll
    for (int it = 0; it < CPR; ++it) {
      const int rr = (64 / CPR) * it + lane / CPR, c = lane % CPR;
      const u32x4_t x = o_chunk_read<CPR>(ot, rr, c);
      const int qi = qbase[rr >> 5] + (rr & 31);
      if (qi < N) *reinterpret_cast<u32x4_t*>(p.o + head + (size_t)qi * D + c * 8) = x;
    }
  }
}

}  // namespace fa
