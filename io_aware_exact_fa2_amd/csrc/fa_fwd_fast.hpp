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
//     staging, no VALU work) into two LDS slots each; one barrier per tile. The copy
//     instructions are spread over the pipeline steps, one per S^T MFMA step, so a
//     wave never stalls on a burst of them. K runs
//     one tile ahead of V: while tile j is finished, the S^T MFMAs of tile j+1 are
//     issued in the same straight-line block as the exponentials of tile j, so the
//     matrix cores and the VALU work on different tiles at the same time. Both stay row-major in LDS; K rows carry one 16-byte pad chunk and V rows
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
//   * Lazy rescale (tau > 0, a kernel argument): the reference max of a row is raised
//     (and O~, l rescaled by alpha) only when a tile's max exceeds it by more than tau
//     in log2 units; otherwise the old reference is kept, so probabilities stay below
//     2^tau. Softmax is invariant to the reference, so O and L are unchanged; tau = 0
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
  static constexpr int K_INSTR = (K_CHUNKS + 63) / 64;  // 1 KB wave copies per tile
  static constexpr int V_INSTR = (V_CHUNKS + 63) / 64;
  static constexpr int K_PER_WAVE = (K_INSTR + NW - 1) / NW;
  static constexpr int V_PER_WAVE = (V_INSTR + NW - 1) / NW;
  static constexpr int LDS = 2 * 16 * (K_CHUNKS + V_CHUNKS);
  static_assert(D == 64 || D == 128, "fast path head dims");
  static_assert(BC % 32 == 0, "key tiles are whole 32-key MFMA blocks");
};

template <bool BF16, int D, bool CAUSAL, int QB, int NW, int BC, int WPE>
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
    koff[ii] = (f < G::K_CHUNKS && ch < G::CPR) ? row * D + ch * 8 : -1;
  }
#pragma unroll
  for (int ii = 0; ii < G::V_PER_WAVE; ++ii) {
    const int i = wid + ii * NW;
    const int f = i * 64 + lane, row = f / G::VPC, ch = f % G::VPC;
    voff[ii] = (f < G::V_CHUNKS && ch < G::CPR) ? row * D + ch * 8 : -1;
  }

  // HBM -> LDS copies of the key (or value) tile j into one LDS slot. Rows past N
  // are clamped to row N-1 (always a valid address); their scores are masked to
  // -inf, so their probabilities are exactly 0 and the duplicated values add nothing.
  auto issue_one = [&](const uint16_t* src, u32x4_t* dst, const int* offs, int n_instr, int ii,
                       int j) {
    const int i = wid + ii * NW;
    if (i < n_instr) {
      const int k0 = j * BC;
      int off = offs[ii];
      if (k0 + BC > N && off >= 0 && k0 + off / D >= N) off = (N - 1 - k0) * D + (off & (D - 1));
      if (off >= 0)
        __builtin_amdgcn_global_load_lds(src + (size_t)k0 * D + off, (lds_void_t*)(dst + i * 64),
                                         16, 0, 0);
    }
  };
  auto issue_k = [&](u32x4_t* dst, int j) {
#pragma unroll
    for (int ii = 0; ii < G::K_PER_WAVE; ++ii) issue_one(kg, dst, koff, G::K_INSTR, ii, j);
  };
  auto issue_v = [&](u32x4_t* dst, int j) {
#pragma unroll
    for (int ii = 0; ii < G::V_PER_WAVE; ++ii) issue_one(vg, dst, voff, G::V_INSTR, ii, j);
  };
  // The copies of one loop iteration, spread one per pipeline step so that a wave
  // never stalls on a burst of copy instructions: K tile jk into k_dst (if jk < n_kt)
  // then V tile jv into v_dst (if jv < n_kt).
  constexpr int NDMA = G::K_PER_WAVE + G::V_PER_WAVE;
  struct Copies {
    u32x4_t* k_dst;
    u32x4_t* v_dst;
    int jk, jv;
  };
  auto copy_step = [&](const Copies& cp, int i) {
    if (i < G::K_PER_WAVE) {
      if (cp.jk < n_kt) issue_one(kg, cp.k_dst, koff, G::K_INSTR, i, cp.jk);
    } else if (i < NDMA) {
      if (cp.jv < n_kt) issue_one(vg, cp.v_dst, voff, G::V_INSTR, i - G::K_PER_WAVE, cp.jv);
    }
  };
  auto copy_all = [&](const Copies& cp) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) copy_step(cp, i);
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

  constexpr int NQK = (BC / 32) * (D / 16);   // K fragments (S^T MFMA steps) per tile
  constexpr int NPV = (D / 32) * (BC / 16);   // V fragments (P V MFMA steps) per tile
  constexpr int SPQ = BC / 2;                 // scores per lane per query block and tile
  constexpr int NSC = SPQ * QB;               // scores per lane per tile
  constexpr int SPS = NSC / NQK;              // scores exponentiated per S^T step
  constexpr int MPS = NSC / NPV;              // scores max-reduced per P V step
  static_assert(SPS % 2 == 0 && NSC % NQK == 0 && NSC % NPV == 0, "pipeline step split");
  typedef f32x16_t STile[BC / 32][QB];        // S^T accumulators of one key tile
  const unsigned char* const ks_base[2] = {reinterpret_cast<const unsigned char*>(ks0) + k_lane,
                                           reinterpret_cast<const unsigned char*>(ks1) + k_lane};
  const unsigned char* const vs_base[2] = {reinterpret_cast<const unsigned char*>(vs0) + v_lane,
                                           reinterpret_cast<const unsigned char*>(vs1) + v_lane};
  // flattened score index e -> (query block e / SPQ, key block, accumulator register)
  auto sc = [](const STile& s, int e) -> float { return s[(e % SPQ) / 16][e / SPQ][e % 16]; };

  // LDS reads of MFMA operands: K fragment of S^T step i, and the two transposed V
  // reads of P V step i (head-dim block db = i / (BC/16), 16-key step st = i % (BC/16))
  auto k_frag = [&](const unsigned char* kb_, int i) {
    const int kb = i / (D / 16), ds = i % (D / 16);
    return *reinterpret_cast<const u32x4_t*>(kb_ + (kb * 32 * G::KPC + 2 * ds) * 16);
  };
  auto v_frag = [&](const unsigned char* vb_, int i) {
    const int db = i / (BC / 16), st = i % (BC / 16);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(vb_ + ((16 * st + 0) * G::VPC + 4 * db) * 16));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(vb_ + ((16 * st + 4) * G::VPC + 4 * db) * 16));
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };
  auto zero = [](STile& s) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
  };

  // plain S^T = K Q^T of one tile (prologue only)
  auto qk_plain = [&](const unsigned char* kb_, STile& s) {
    zero(s);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int kb = i / (D / 16), ds = i % (D / 16);
      const u32x4_t kf = k_frag(kb_, i);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = E::mfma(kf, qf[qb][ds], s[kb][qb]);
    }
  };

  // -inf on keys past N and, under the causal mask, on keys after the query; only
  // tiles that reach past N or cross the diagonal need it
  auto mask = [&](STile& s, int j) {
    const int k0 = j * BC;
    const bool masked = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > wq0);
    if (!masked) return;
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
        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
    }
  };

  // p = exp2(s*c - m*c) for flattened scores [e0, e0+n); consecutive pairs are packed
  // into the P V operand of their query block: 16-key step (e % SPQ) / 8, word (e % 8) / 2
  u32x4_t pb[BC / 16][QB];
  float lsum[QB][2];
  auto exp_scores = [&](const STile& s, int e0, int n) {
#pragma unroll
    for (int e = e0; e < e0 + n; e += 2) {
      const int qb = e / SPQ;
      const float msc = ms[qb];
      // c > 0 on this path, so a masked score (-inf) gives exp2(-inf) = 0 exactly
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc(s, e), c, -msc));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc(s, e + 1), c, -msc));
      lsum[qb][0] += p0;
      lsum[qb][1] += p1;
      pb[(e % SPQ) / 8][qb][(e % 8) / 2] = E::pack(p0, p1);
    }
  };

  // Block B: S^T of tile j+1 (MFMA) interleaved with the exponentials of tile j (VALU);
  // K fragments are read two steps ahead
  auto qk_exp = [&](const unsigned char* kb_, STile& s_next, const STile& s_cur,
                    const Copies& cp) {
    zero(s_next);
    u32x4_t kf0 = k_frag(kb_, 0), kf1 = k_frag(kb_, 1);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const u32x4_t kf2 = (i + 2 < NQK) ? k_frag(kb_, i + 2) : kf1;
      const int kb = i / (D / 16), ds = i % (D / 16);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s_next[kb][qb] = E::mfma(kf0, qf[qb][ds], s_next[kb][qb]);
      exp_scores(s_cur, i * SPS, SPS);
      copy_step(cp, i);
      kf0 = kf1;
      kf1 = kf2;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Block C: P V of tile j (MFMA) interleaved with the row max of tile j+1 (VALU)
  float mxn[QB][2];
  auto pv_max = [&](const unsigned char* vb_, const STile& s_next) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mxn[qb][0] = mxn[qb][1] = -__builtin_inff();
    u32x4_t vf0 = v_frag(vb_, 0), vf1 = v_frag(vb_, 1);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const u32x4_t vf2 = (i + 2 < NPV) ? v_frag(vb_, i + 2) : vf1;
      const int db = i / (BC / 16), st = i % (BC / 16);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = E::mfma(vf0, pb[st][qb], oacc[db][qb]);
#pragma unroll
      for (int e = i * MPS; e < (i + 1) * MPS; ++e)
        mxn[e / SPQ][e & 1] = __builtin_fmaxf(mxn[e / SPQ][e & 1], sc(s_next, e));
      vf0 = vf1;
      vf1 = vf2;
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One key tile j whose masked S^T is in s_cur and whose max is already folded into
  // ms: exponentials and P V of tile j, overlapped with the S^T, mask and max of tile
  // j+1 (from K slot k_next). On a wave's last tile the look-ahead reads a stale but
  // valid K slot and its result is dropped (`next` false: no max update).
  static_assert(NDMA <= NQK, "copies fit in the S^T pipeline steps");
  auto tile = [&](const STile& s_cur, STile& s_next, int k_next, int v_cur, int j, bool next,
                  const Copies& cp) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lsum[qb][0] = lsum[qb][1] = 0.f;
    qk_exp(ks_base[k_next], s_next, s_cur, cp);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_part[qb] += lsum[qb][0] + lsum[qb][1];
    mask(s_next, j + 1);
    pv_max(vs_base[v_cur], s_next);
    if (next) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        grow_max(qb, xhalf_max(__builtin_fmaxf(mxn[qb][0], mxn[qb][1])) * c);
    }
  };

  // row max of a tile in log2 units (prologue)
  auto first_max = [&](const STile& s) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[kb][qb][r]);
      ms[qb] = xhalf_max(mx) * c;  // tile 0 holds key 0, allowed for every row: finite
    }
  };

  // ---- main loop ---------------------------------------------------------------------
  // Slots: K tile t lives in ks[t % 2], V tile t in vs[t % 2]. While tile j is being
  // finished (V_j in vs[j%2]) the S^T of tile j+1 is computed from ks[(j+1)%2], and
  // the copies of K_{j+2} (into ks[j%2]) and V_{j+1} (into vs[(j+1)%2]) are in flight.
  STile sa, sb;
  issue_k(ks0, 0);
  issue_v(vs0, 0);
  if (n_kt > 1) issue_k(ks1, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (wave_live) {
    qk_plain(ks_base[0], sa);
    mask(sa, 0);
    first_max(sa);
  }
  __syncthreads();  // every wave is done with ks0 before K_2 overwrites it
  for (int j = 0; j < n_kt; j += 2) {
    const Copies ce = {ks0, vs1, j + 2, j + 1};
    if (wave_live && j < w_kt) tile(sa, sb, 1, 0, j, j + 1 < w_kt, ce);
    else copy_all(ce);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 >= n_kt) break;
    const Copies co = {ks1, vs0, j + 3, j + 2};
    if (wave_live && j + 1 < w_kt) tile(sb, sa, 0, 1, j + 1, j + 2 < w_kt, co);
    else copy_all(co);
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
