// fa_bwd_wide.hpp — the dK/dV and dQ kernels of the backward for gfx950 at head dims 64
// and 128: one workgroup per 128 keys (dK/dV) or 128 queries (dQ), 32 per wave, the other
// side's rows streamed in 32-row blocks through a ring of LDS slots, and each block's
// products and softmax terms in a three-stage pipeline of fenced MFMA slots.
//
// What they compute is the chain rule of fa_bwd.hpp ([P1] currybab.bearblog.dev, FA2
// section: the backward recomputes P_ij = exp(S_ij - L_i) block by block from the saved
// L instead of storing P). dK/dV: for the wave's 32 keys (on the lanes) and every query
// block,
//     S = Q K^T, dP = dO V^T, P = exp2(S c - L log2 e), dS = P (dP - D),
//     dV^T += dO^T P,  dK^T += Q^T dS,
// and at the end dK = scale dK. D_i = rowsum(dO * O)_i and L_i log2(e) come from the
// D pass (fa_bwd_delta_kernel). dQ: see fa_bwd_dq_wide_kernel below.
//
// Why these kernels. The kernels of fa_bwd.hpp left the order of their products and LDS
// operand reads to the compiler, and each product waited for a read issued just before
// it: the dK/dV matrix core was busy about a third of the time at the chip's full clock.
// Here dK/dV iteration t issues, one MFMA per slot, the dV/dK products of query block t
// (16 at d = 128), then the S/dP products of block t+2 (16), and between them the softmax
// terms of block t+1 (80 VALU ops per lane, spread over the slots by a compile-time
// table); every operand read runs FA_BW_PF steps ahead of its product and the wave waits
// for LDS once per two steps. Block b's rows reach LDS by buffer-to-LDS copies issued in
// iteration b-5 into ring slot b % 6 (Q and dO: 16 KB at d = 128), with its L log2(e) and
// D (256 bytes each); one barrier per iteration.
//
// Rows past N need no mask: their copies read zeros (Q, dO, L and D), so S = dP = 0,
// P = 1 and dS = 0, and they add dO^T P = 0 and Q^T dS = 0. Keys past N (lanes) compute
// columns that are not stored. Under the causal mask, a block that reaches past the
// wave's first key gets S = -inf (c > 0; +inf when c < 0) above the diagonal, so P = 0
// and dS = 0 there; c = 0 takes the kernels of fa_bwd.hpp.
#pragma once

#include "fa_bwd.hpp"

#ifndef FA_BW_PF
#define FA_BW_PF 3  // MFMA steps an LDS operand read runs ahead
#endif
#ifndef FA_BW_PAIR
#define FA_BW_PAIR 1  // one LDS wait per two MFMA steps
#endif

namespace fa {

// The softmax terms of one 32-query block, as a stream of VALU ops placed into the MFMA
// slots of an iteration. A lane holds 16 scores (registers r = 0..15, queries
// key_of_reg(r, half)); pair v holds registers 2v and 2v+1. Per pair: ops 0-1 the
// exponent arguments s c - L2 (FMA), 2-3 their exponentials, 4-5 dP - D, 6-7 the
// products P (dP - D), 8 the 16-bit pack of P, 9 that of dS. The stages of consecutive
// pairs are staggered (step k: ops 0, 1, 4, 5 of pair k, exponentials of pair k-1, the
// products and the P pack of pair k-2, the dS pack of pair k-3), and the stream goes
// into slots first .. NSLOT-1 so that the estimated issue time of every slot (its ops,
// MFMA, reads and copies, in half-cycles) is as even as possible.
struct BwdOpSched {
  int code[80];  // 10 * pair + op
  int n;
  int first[65];  // ops [first[s], first[s + 1]) go into slot s
};
template <int NSLOT, int FIRST, int PF, int NC, int NAS>
constexpr BwdOpSched make_bwd_op_sched(bool two_blocks) {
  // two_blocks: NSLOT = 2 NAS dV/dK slots, then the S/dP slots; else S/dP slots only
  BwdOpSched t{};
  int n = 0;
  const int ops_of[4][4] = {{0, 1, 4, 5}, {2, 3, -1, -1}, {6, 7, 8, -1}, {9, -1, -1, -1}};
  for (int k = 0; k < 8 + 3; ++k)
    for (int st = 0; st < 4; ++st) {
      const int v = k - st;
      if (v < 0 || v >= 8) continue;
      for (int q = 0; q < 4 && ops_of[st][q] >= 0; ++q) t.code[n++] = 10 * v + ops_of[st][q];
    }
  t.n = n;
  const int op_cost[10] = {11, 11, 24, 24, 10, 10, 10, 10, 11, 11};
  int fixed[64] = {};
  long total = 0;
  for (int sl = 0; sl < NSLOT; ++sl) {
    int f = 4;  // the MFMA
    const int nbs = two_blocks ? (NSLOT - 2 * NAS) / 2 : NSLOT / 2;  // S/dP steps
    if (two_blocks && sl < 2 * NAS) {  // dV/dK block: transposed reads, L/D reads, copies
      const int i = sl / 2;
      f += (i + PF < NAS) ? 40 : 8;
      if (sl < 2) f += 32;
      if (sl % 2 == 1 && sl / 2 < NC) f += 18;
    } else {  // S/dP block: row reads, the next iteration's transposed reads
      const int i = (two_blocks ? sl - 2 * NAS : sl) / 2;
      f += (i + PF < nbs) ? 8 : (two_blocks ? 40 : 0);
    }
    fixed[sl] = f;
    total += f;
  }
  long ops_total = 0;
  for (int i = 0; i < n; ++i) ops_total += op_cost[t.code[i] % 10];
  total += ops_total;
  long cum = 0;
  int o = 0;
  for (int sl = 0; sl < NSLOT; ++sl) {
    t.first[sl] = o;
    cum += fixed[sl];
    if (sl < FIRST) continue;
    const long target = total * (sl + 1) / NSLOT;
    while (o < n) {
      const int c = op_cost[t.code[o] % 10];
      if (cum + c <= target || (cum + c - target) < (target - cum)) {
        cum += c;
        ++o;
      } else {
        break;
      }
    }
  }
  t.first[NSLOT] = n;
  return t;
}
// the loop: 2 NAS + 2 NBS slots, ops from slot 3 (the block's L and D are read in slots 0
// and 1); the prologue: the 2 NBS S/dP slots of block 1 carry the softmax of block 0
template <int PF, int NC, int NAS, int NBS>
constexpr BwdOpSched kBwdLoopOps = make_bwd_op_sched<2 * NAS + 2 * NBS, 3, PF, NC, NAS>(true);
template <int PF, int NC, int NAS, int NBS>
constexpr BwdOpSched kBwdPrologueOps = make_bwd_op_sched<2 * NBS, 2, PF, NC, NAS>(false);

// waves per SIMD that the slot-scheduled backward kernels are compiled for: one, except
// dQ at head dim 64, which fits two in 256 registers (dK/dV at 64 does not: bounded to two
// waves it crashed the compiler's AGPR-copy rewrite)
template <int D> constexpr int kBwdWavesKV = 1;
template <int D> constexpr int kBwdWavesQ = D == 64 ? 2 : 1;

// x = (c >= lo) ? x : m, with c a constant after unrolling (m from a register)
__device__ __forceinline__ float keep_if_ge(float x, int c, int lo, float m) {
  asm("v_cmp_ge_i32 vcc, %2, %1\n\tv_cndmask_b32 %0, %3, %0, vcc"
      : "+v"(x) : "v"(lo), "n"(c), "v"(m) : "vcc");
  return x;
}

template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kBwdWavesKV<D>, kBwdWavesKV<D>)))
fa_bwd_dkdv_wide_kernel(const BwdParams p) {
  using E = Elt<BF16>;
  constexpr int CPR = D / 8, NDS = D / 16, NDB = D / 32, NW = 4, QB = 32, R = 6;
  constexpr int SLOT = QB * CPR;  // 16-byte chunks of one block's Q (or dO) rows
  constexpr int PPW = SLOT / 64 / NW;  // 1 KB pieces per wave, block and tensor
  constexpr int NAS = 2 * NDB;    // dV/dK steps (two products each) per block
  constexpr int PF = FA_BW_PF;
  constexpr int NC = 1 + 2 * PPW; // copies per wave and block: L2 or D, then Q, then dO
  static_assert(D == 64 || D == 128, "head dims");
  static_assert(PF <= NAS && PF <= NDS && NC <= NAS, "read-ahead and copies fit the blocks");
  constexpr int AHEAD = 5;        // block t + AHEAD is copied in iteration t
  static_assert(PF >= 1 && 4 * PF <= 15, "operand reads a few steps ahead (lgkmcnt holds 15)");
  static_assert(R % 2 == 0 && R >= AHEAD + 1, "ring: even (tile buffers alternate) and deep enough");
  __shared__ __attribute__((aligned(1024))) u32x4_t qring[R * SLOT];
  __shared__ __attribute__((aligned(1024))) u32x4_t dring[R * SLOT];
  __shared__ __attribute__((aligned(256))) float lring[R * 64];  // L log2(e) of each slot's rows
  __shared__ __attribute__((aligned(256))) float dlring[R * 64]; // D of each slot's rows

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N;
  const int n_kt = (N + 127) / 128;
  int bh, kt;
  tile_order<CAUSAL>(blockIdx.x, p.BH, n_kt, bh, kt);  // the first key tile sees the most queries
  const size_t head = (size_t)bh * (size_t)N * D;
  const int k0 = kt * 128, kw = k0 + 32 * wid, kj = kw + l32;
  const int g0 = CAUSAL ? k0 / QB : 0;      // queries before k0 never see these keys
  const int nb = (N + QB - 1) / QB - g0;    // query blocks of this work item (>= 1)
  const float c = p.c;
  const float s_mask = c > 0.f ? -__builtin_inff() : __builtin_inff();

  // K and V of the wave's 32 keys as B operands (lane: key kj, columns 16 ds + 8 hh ..),
  // in AGPRs for the whole loop; keys past N load row N - 1 (their columns are not stored)
  u32x4_t kf[NDS], vf[NDS];
  {
    const int kr = min(kj, N - 1);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const size_t off = head + (size_t)kr * D + ds * 16 + hh * 8;
      kf[ds] = ld16(p.k + off);
      vf[ds] = ld16(p.v + off);
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      asm volatile("" : "+a"(kf[ds]));
      asm volatile("" : "+a"(vf[ds]));
    }
  }
  f32x16_t dk[D / 32], dv[D / 32];  // dK^T, dV^T: rows = head dims, lane = key; in AGPRs
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  // ---- copies: block g (rows 32 g ..) into ring slot sl. Copy 0 moves 64 floats of L
  // log2(e) (even waves) or of D (odd waves) from row 32 g on (the second 32 are not
  // read; a pair of waves copies the same bytes); copies 1 .. PPW move 1 KB pieces wid,
  // wid + 4, .. of the Q rows, the next PPW those of the dO rows: lane l of piece c
  // writes chunk 64 c + l of the slot and fetches the logical chunk the swizzle puts
  // there. ---------------------------------------------------------------------------
  uint32_t cvoff[PPW];
#pragma unroll
  for (int cc = 0; cc < PPW; ++cc) {
    const int f = (wid + NW * cc) * 64 + lane, row = f / CPR, ph = f % CPR;
    cvoff[cc] = (uint32_t)(row * D + (ph ^ swz_b<D>(row)) * 8) * 2u;
  }
  const uint32_t q_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(qring + wid * 64));
  const uint32_t d_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dring + wid * 64));
  const float* ld_src = (wid & 1) ? p.delta : p.lse2;
  const uint32_t ld_lds = __builtin_amdgcn_readfirstlane(
      (wid & 1) ? (uint32_t)(uintptr_t)dlring : (uint32_t)(uintptr_t)lring);
  auto copy = [&](int g, int sl, int cc) __attribute__((always_inline)) {
    const int row0 = g * QB;
    const int left = N - row0;  // rows of the block below N (may be <= 0)
    if (cc == 0) {
      const uint32_t n4 = sclamp(left, 64) * 4u;
      lds_copy4(buffer_rsrc((uint64_t)(uintptr_t)(ld_src + (size_t)bh * N + row0), n4),
                (uint32_t)lane * 4u, ld_lds, sl * 256);
    } else {
      const uint32_t nb2 = sclamp(left, QB) * (uint32_t)(D * 2);
      const int piece = (cc - 1) % PPW;
      const bool is_q = cc <= PPW;
      const uint16_t* src = (is_q ? p.q : p.dout) + head + (size_t)row0 * D;
      lds_copy16(buffer_rsrc((uint64_t)(uintptr_t)src, nb2), cvoff[piece], is_q ? q_lds : d_lds,
                 sl * SLOT * 16 + piece * NW * 1024);
    }
  };

  // ---- per-lane LDS read addresses ---------------------------------------------------
  // Row operand (A = 32 rows x 16 columns of a block): MFMA row m reads block row
  // key_of_row(m), logical chunk 2 ds + hh (the ds step folds in by XOR: the swizzle
  // permutes the 16 chunks of a 256-byte row).
  // The addresses include the ring's base and are held opaque, so that every read of a
  // slot is one of them plus a constant offset (the slots of the second ring lie past
  // the 64 KB reach of that offset).
  uint32_t raddr[2][NDS];  // [w: Q, dO][ds]
  {
    const int row = key_of_row(l32);
    const uint32_t r = (uint32_t)((row * CPR + (hh ^ swz_b<D>(row))) * 16);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      raddr[0][ds] = (uint32_t)(uintptr_t)qring + (r ^ (uint32_t)(ds << 5));
      raddr[1][ds] = (uint32_t)(uintptr_t)dring + (r ^ (uint32_t)(ds << 5));
      asm volatile("" : "+v"(raddr[0][ds]), "+v"(raddr[1][ds]));
    }
  }
  uint32_t taddr[2][NDB][2];  // [w: dO, Q][db][h]
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t o = bwd_tr_off<D>(lane, db, h);
      taddr[0][db][h] = (uint32_t)(uintptr_t)dring + o;
      taddr[1][db][h] = (uint32_t)(uintptr_t)qring + o;
      asm volatile("" : "+v"(taddr[0][db][h]), "+v"(taddr[1][db][h]));
    }
  typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
  typedef __attribute__((address_space(3))) const f32x4_t lds_f32x4_t;
  // rows of block slot sl, columns 16 ds .. (w 0: Q, 1: dO)
  auto row_op = [&](int w, int sl, int ds) __attribute__((always_inline)) {
    return *(lds_u32x4_t*)(uintptr_t)(raddr[w][ds] + (uint32_t)(sl * SLOT * 16));
  };
  // transposed operand of step i (16-query half i / NDB, head dims 32 (i % NDB) ..) of
  // block slot sl (w 0: dO, 1: Q): rows 16 (i / NDB) .., two 4-row halves
  auto tr_op = [&](int w, int sl, int i) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)(sl * SLOT * 16 + (i / NDB) * 16 * CPR * 16);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(uintptr_t)(taddr[w][i % NDB][0] + off));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(uintptr_t)(taddr[w][i % NDB][1] + off));
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };
  // L log2(e) and D of registers 4 g .. 4 g + 3 (queries 16 (g >> 1) + 8 hh + 4 (g & 1) ..)
  auto ld_op = [&](const float* ring, int sl, int g) __attribute__((always_inline)) {
    const int ql = 16 * (g >> 1) + 8 * hh + 4 * (g & 1);
    return *(lds_f32x4_t*)(uintptr_t)((uint32_t)(uintptr_t)(ring + sl * 64 + ql));
  };

  // ---- the softmax terms of one block: the op stream --------------------------------
  float xq[2][2], dq3[3][2], pq[2][2], eq[2][2];  // values of the pairs in flight
  auto soft_op = [&](const BwdOpSched& sch, const f32x16_t& s, const f32x16_t& dp,
                     const f32x4_t (&lv)[4], const f32x4_t (&dv4)[4], u32x4_t (&pop)[2],
                     u32x4_t (&dsop)[2], int o) __attribute__((always_inline)) {
    const int v = sch.code[o] / 10, op = sch.code[o] % 10;
    const int r0 = 2 * v;
    if (op < 2) {
      const int r = r0 + op;
      xq[v % 2][op] = __builtin_fmaf(s[r], c, -lv[r / 4][r % 4]);
      asm volatile("" : "+v"(xq[v % 2][op]));
    } else if (op < 4) {
      pq[v % 2][op - 2] = __builtin_amdgcn_exp2f(xq[v % 2][op - 2]);
      asm volatile("" : "+v"(pq[v % 2][op - 2]));
    } else if (op < 6) {
      const int e = op - 4, r = r0 + e;
      dq3[v % 3][e] = dp[r] - dv4[r / 4][r % 4];
      asm volatile("" : "+v"(dq3[v % 3][e]));
    } else if (op < 8) {
      const int e = op - 6;
      eq[v % 2][e] = pq[v % 2][e] * dq3[v % 3][e];
      asm volatile("" : "+v"(eq[v % 2][e]));
    } else {
      const float* src = op == 8 ? pq[v % 2] : eq[v % 2];
      uint32_t w = E::pack(src[0], src[1]);
      asm volatile("" : "+v"(w));
      (op == 8 ? pop : dsop)[r0 / 8][(r0 % 8) / 2] = w;
    }
  };

  // ---- causal mask of a fresh S tile (block g): s = s_mask where the query precedes
  // the lane's key; only blocks that start before the wave's last key need it --------
  auto mask = [&](f32x16_t& s, int g) __attribute__((always_inline)) {
    if (!CAUSAL || g * QB >= kw + 31) return;
    // wait out the S products before the inline-assembly compares read them
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
    const int lo = kj - (g * QB + 8 * hh);  // register r keeps when key_of_reg(r, 0) >= lo
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = keep_if_ge(s[r], key_of_reg(r, 0), lo, s_mask);
  };
  auto zero16 = [](f32x16_t& x) {
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = 0.f;
  };

  // ---- one iteration: dV, dK of block t; softmax terms of block t+1; S, dP of block t+2
  constexpr BwdOpSched OPS = kBwdLoopOps<PF, NC, NAS, NDS>;
  u32x4_t anext[PF][2];  // the first transposed operands of the next iteration
  auto iteration = [&](int u, int t, f32x16_t& s_new, f32x16_t& dp_new, const f32x16_t& s_mid,
                       const f32x16_t& dp_mid, u32x4_t (&p_mid)[2], u32x4_t (&ds_mid)[2],
                       const u32x4_t (&p_cur)[2], const u32x4_t (&ds_cur)[2])
      __attribute__((always_inline)) {
    // ring slots: block t in slot u = t % R
    const int sl0 = u, sl1 = (u + 1) % R, sl2 = (u + 2) % R, slc = (u + AHEAD) % R;
    f32x4_t lv[4], dv4[4];
    u32x4_t aop[NAS][2], bop[NDS][2];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      aop[i][0] = anext[i][0];
      aop[i][1] = anext[i][1];
    }
    // dV^T += dO^T P and dK^T += Q^T dS of block t: step i (16-query half i / NDB,
    // head-dim block i % NDB), slot w = 0: dV, 1: dK
#pragma unroll
    for (int sa = 0; sa < 2 * NAS; ++sa) {
      const int i = sa / 2, w = sa % 2, hq = i / NDB, db = i % NDB;
      // keep the previous step's sources live until this step (the inline-assembly MFMAs
      // read them over several cycles)
      if (w == 0 && i > 0)
        asm volatile("" ::"v"(aop[i - 1][0]), "v"(aop[i - 1][1]), "v"(p_cur[(i - 1) / NDB]),
                     "v"(ds_cur[(i - 1) / NDB]));
#if FA_BW_PAIR
      // one LDS wait per two steps: the operands of steps i and i + 1 together
      if (w == 0 && i % 2 == 0)
        asm volatile("" ::"v"(aop[i][0]), "v"(aop[i][1]), "v"(aop[i + 1][0]), "v"(aop[i + 1][1]));
#endif
      if (w == 0) mfma_acc_agpr<BF16>(dv[db], aop[i][0], p_cur[hq]);
      else mfma_acc_agpr<BF16>(dk[db], aop[i][1], ds_cur[hq]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + PF < NAS) aop[i + PF][w] = tr_op(w, sl0, i + PF);
      else bop[i + PF - NAS][w] = row_op(w, sl2, i + PF - NAS);
      if (sa == 0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) lv[g] = ld_op(lring, sl1, g);
      } else if (sa == 1) {
#pragma unroll
        for (int g = 0; g < 4; ++g) dv4[g] = ld_op(dlring, sl1, g);
      }
      if (w == 1 && i < NC) copy(g0 + t + AHEAD, slc, i);
#pragma unroll
      for (int o = OPS.first[sa]; o < OPS.first[sa + 1]; ++o)
        soft_op(OPS, s_mid, dp_mid, lv, dv4, p_mid, ds_mid, o);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"v"(aop[NAS - 1][0]), "v"(aop[NAS - 1][1]), "v"(p_cur[1]), "v"(ds_cur[1]));
    // S = Q K^T and dP = dO V^T of block t+2: step i (16 head dims), slot w = 0: S, 1: dP
    zero16(s_new);
    zero16(dp_new);
#pragma unroll
    for (int sb = 0; sb < 2 * NDS; ++sb) {
      const int i = sb / 2, w = sb % 2;
#if FA_BW_PAIR
      if (w == 0 && i % 2 == 0) {
        asm volatile("" ::"v"(bop[i][0]), "v"(bop[i][1]), "v"(bop[i + 1][0]), "v"(bop[i + 1][1]));
        __builtin_amdgcn_sched_barrier(0);  // (the product must not move above the wait)
      }
#endif
      if (w == 0) s_new = E::mfma(bop[i][0], kf[i], s_new);
      else dp_new = E::mfma(bop[i][1], vf[i], dp_new);
      __builtin_amdgcn_sched_barrier(0);
      if (i + PF < NDS) bop[i + PF][w] = row_op(w, sl2, i + PF);
      else anext[i + PF - NDS][w] = tr_op(w, sl1, i + PF - NDS);
#pragma unroll
      for (int o = OPS.first[2 * NAS + sb]; o < OPS.first[2 * NAS + sb + 1]; ++o)
        soft_op(OPS, s_mid, dp_mid, lv, dv4, p_mid, ds_mid, o);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask(s_new, g0 + t + 2);
  };

  // ---- prologue: blocks 0 .. 4 copied; S, dP of block 0; its softmax terms with the S,
  // dP of block 1 ------------------------------------------------------------------------
#pragma unroll
  for (int b = 0; b < AHEAD; ++b)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) copy(g0 + b, b, cc);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((AHEAD - 2) * NC) : "memory");  // blocks 0, 1
  __syncthreads();
  f32x16_t sA, sB, dA, dB;       // S and dP of even and odd blocks
  u32x4_t pA[2], pB[2], dsA[2], dsB[2];  // P and dS operands of even and odd blocks
  {
    zero16(sA);
    zero16(dA);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      sA = E::mfma(row_op(0, 0, ds), kf[ds], sA);
      dA = E::mfma(row_op(1, 0, ds), vf[ds], dA);
    }
    mask(sA, g0);
    f32x4_t lv[4], dv4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      lv[g] = ld_op(lring, 0, g);
      dv4[g] = ld_op(dlring, 0, g);
    }
    constexpr BwdOpSched POPS = kBwdPrologueOps<PF, NC, NAS, NDS>;
    u32x4_t bq[NDS][2];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      bq[i][0] = row_op(0, 1, i);
      bq[i][1] = row_op(1, 1, i);
    }
    zero16(sB);
    zero16(dB);
#pragma unroll
    for (int sb = 0; sb < 2 * NDS; ++sb) {
      const int i = sb / 2, w = sb % 2;
      if (w == 0) sB = E::mfma(bq[i][0], kf[i], sB);
      else dB = E::mfma(bq[i][1], vf[i], dB);
      __builtin_amdgcn_sched_barrier(0);
      if (i + PF < NDS) bq[i + PF][w] = row_op(w, 1, i + PF);
#pragma unroll
      for (int o = POPS.first[sb]; o < POPS.first[sb + 1]; ++o)
        soft_op(POPS, sA, dA, lv, dv4, pA, dsA, o);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask(sB, g0 + 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // blocks 2 .. 4
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    anext[i][0] = tr_op(0, 0, i);
    anext[i][1] = tr_op(1, 0, i);
  }

  // ---- main loop, unrolled over the ring: S/dP tiles and P/dS operands alternate
  // between the even (A) and odd (B) buffers; with R even the parity of t is that of u --
  for (int t0 = 0; t0 < nb; t0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int t = t0 + u;
      if (t >= nb) break;
      if (u % 2 == 0) iteration(u, t, sA, dA, sB, dB, pB, dsB, pA, dsA);
      else iteration(u, t, sB, dB, sA, dA, pA, dsA, pB, dsB);
      // every copy but this iteration's has landed (the next iteration reads block t+3's
      // rows, block t+2's L and D); the barrier follows this wave's last read of block
      // t's slot, which the next iteration's copies refill (its 4 PF transposed reads of
      // block t+1 may stay in flight)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NC) : "memory");
      asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(4 * PF) : "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- dK = scale dK, dV: rows kj < N --------------------------------------------------
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dk[db]), "+a"(dv[db]));
  }
  if (kj < N) {
    bwd_store_rows<BF16, D>(p.dk + head, dk, kj, hh, p.scale);
    bwd_store_rows<BF16, D>(p.dv + head, dv, kj, hh, 1.0f);
  }
}

}  // namespace fa

namespace fa {

// ---- dQ ------------------------------------------------------------------------------
// One workgroup per 128 query rows (32 per wave); the keys stream in 32-key blocks
// through a ring of LDS slots (K and V rows, 16 KB per block at d = 128). For the wave's
// queries (on the lanes) and every key block,
//     S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), P^T = exp2(S^T c - L log2 e),
//     dQ^T += K^T dS^T,
// and at the end dQ = scale dQ. Iteration t issues the dQ products of key block t (8 at
// d = 128), then the S/dP products of block t+2 (16), and between them the softmax terms
// of block t+1 (72 VALU ops per lane: L and D are the lane's own). An MFMA slot's operand is read
// FA_BQ_PS slots ahead, and the wave waits for LDS once per two slots. Block b is copied
// in iteration b-5 into slot b % 6; one barrier per iteration.
//
// Keys past N need no mask: their K and V rows read as zeros, so dS^T may be nonzero
// there but meets a zero K^T column. Queries past N (lanes) are computed on row N - 1 and
// not stored. Under the causal mask, scores of keys after the lane's query are set to
// the infinity that gives P = 0 (c != 0; c = 0 takes the kernel of fa_bwd.hpp).
#ifndef FA_BQ_PS
#define FA_BQ_PS 6  // operand slots an operand read runs ahead
#endif


// The softmax terms of the wave's query blocks for one key block, 9 ops per pair of
// registers (2v, 2v+1 of query block v / 8): 0-1 FMA, 2-3 exponentials, 4-5 dP - D, 6-7
// the products, 8 the 16-bit pack of dS; staged as in make_bwd_op_sched and spread over
// the MFMA slots (NA dQ operand slots, then the S/dP operand slots, NQB products each) by
// estimated issue time.
struct DqOpSched {
  int code[144];  // 10 * pair + op
  int n;
  int first[49];
};
template <int PS, int NC, int NA, int NOP, int NQB>
constexpr DqOpSched make_dq_op_sched() {
  DqOpSched t{};
  int n = 0;
  const int np = 8 * NQB;
  const int ops_of[4][4] = {{0, 1, 4, 5}, {2, 3, -1, -1}, {6, 7, -1, -1}, {8, -1, -1, -1}};
  for (int k = 0; k < np + 3; ++k)
    for (int st = 0; st < 4; ++st) {
      const int v = k - st;
      if (v < 0 || v >= np) continue;
      for (int q = 0; q < 4 && ops_of[st][q] >= 0; ++q) t.code[n++] = 10 * v + ops_of[st][q];
    }
  t.n = n;
  const int op_cost[9] = {11, 11, 24, 24, 10, 10, 10, 10, 11};
  constexpr int NSL = NOP * NQB;
  int fixed[48] = {};
  long total = 0;
  for (int sl = 0; sl < NSL; ++sl) {
    const int so = sl / NQB;  // operand slot
    int f = 4;
    if (sl % NQB == 0) {
      const int rd = so + PS;  // the operand slot whose operand is read here
      f += (rd < NA || rd >= NOP) ? 40 : 8;
      if (so < NA && so % 2 == 1 && so / 2 < NC) f += 18;
    }
    fixed[sl] = f;
    total += f;
  }
  for (int i = 0; i < n; ++i) total += op_cost[t.code[i] % 10];
  long cum = 0;
  int o = 0;
  for (int sl = 0; sl < NSL; ++sl) {
    t.first[sl] = o;
    cum += fixed[sl];
    const long target = total * (sl + 1) / NSL;
    while (o < n) {
      const int c = op_cost[t.code[o] % 10];
      if (cum + c <= target || (cum + c - target) < (target - cum)) {
        cum += c;
        ++o;
      } else {
        break;
      }
    }
  }
  t.first[NSL] = n;
  return t;
}
template <int PS, int NC, int NA, int NOP, int NQB>
constexpr DqOpSched kDqOps = make_dq_op_sched<PS, NC, NA, NOP, NQB>();

template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kBwdWavesQ<D>, kBwdWavesQ<D>)))
fa_bwd_dq_wide_kernel(const BwdParams p) {
  using E = Elt<BF16>;
  constexpr int CPR = D / 8, NDS = D / 16, NDB = D / 32, NW = 4, KB = 32, R = 6, AHEAD = 5;
  constexpr int NQB = kDqBlocks<D>;
  constexpr int QW = NW * 32 * NQB;  // queries per workgroup
  constexpr int SLOT = KB * CPR;  // 16-byte chunks of one block's K (or V) rows
  constexpr int PPW = SLOT / 64 / NW;  // 1 KB pieces per wave, block and tensor
  constexpr int NC = 2 * PPW;     // copies per wave and block: K, then V
  constexpr int NA = 2 * NDB;     // dQ operand slots per iteration (then NDS x (K, V))
  constexpr int NOP = NA + 2 * NDS;
  constexpr int PS = FA_BQ_PS < NA ? FA_BQ_PS : NA;
  static_assert(D == 64 || D == 128, "head dims");
  static_assert(NQB == 1 || NQB == 2, "one or two query blocks per wave");
  static_assert(NC <= NA / 2 && NOP % 2 == 0, "copies fit the dQ slots");
  static_assert(PS >= 2 && 2 * PS <= 15 && PS % 2 == 0,
                "operands read a few (even) slots ahead (lgkmcnt holds 15)");
  static_assert(R % 2 == 0 && R >= AHEAD + 1, "ring: even and deep enough");
  __shared__ __attribute__((aligned(1024))) u32x4_t kring[R * SLOT];
  __shared__ __attribute__((aligned(1024))) u32x4_t vring[R * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N;
  const int n_qt = (N + QW - 1) / QW;
  int bh, rank;
  tile_order<CAUSAL>(blockIdx.x, p.BH, n_qt, bh, rank);
  const int qt = CAUSAL ? n_qt - 1 - rank : rank;  // the last query tile sees the most keys
  const size_t head = (size_t)bh * (size_t)N * D;
  const int q0 = qt * QW;
  // wave w owns query block w (and 2 NW - 1 - w with two per wave), so that under the
  // causal mask the waves of a workgroup end within a key block of each other
  int qbase[NQB], qi[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    qbase[qb] = q0 + 32 * (qb == 0 ? wid : 2 * NW - 1 - wid);
    qi[qb] = qbase[qb] + l32;
  }
  const int nb = CAUSAL ? (min(q0 + QW, N) + KB - 1) / KB : (N + KB - 1) / KB;
  const float c = p.c;
  const float s_mask = c > 0.f ? -__builtin_inff() : __builtin_inff();

  // Q and dO as B operands (lane: query, columns 16 ds + 8 hh ..), in AGPRs; D_i from dO
  // and O; L_i log2(e); rows past N load row N - 1 and are never stored
  u32x4_t qf[NQB][NDS], dof[NQB][NDS];
  float Dq[NQB], L2[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qr = min(qi[qb], N - 1);
    float dpart = 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const size_t off = head + (size_t)qr * D + ds * 16 + hh * 8;
      qf[qb][ds] = ld16(p.q + off);
      dof[qb][ds] = ld16(p.dout + off);
      const u32x4_t of = ld16(p.o + off);
#pragma unroll
      for (int w = 0; w < 4; ++w) dpart = E::dot2(dof[qb][ds][w], of[w], dpart);
    }
    Dq[qb] = xhalf_sum(dpart);
    L2[qb] = p.lse[(size_t)bh * N + qr] * 1.4426950408889634f;
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) asm volatile("" : "+a"(qf[qb][ds]), "+a"(dof[qb][ds]));
  f32x16_t dq[NQB][NDB];  // dQ^T: rows = head dims, lane = query; in AGPRs
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[qb][db][r] = 0.f;

  // ---- copies: block g (keys 32 g ..) into ring slot sl: copies 0 .. PPW - 1 move 1 KB
  // pieces wid, wid + 4, .. of the K rows, the next PPW those of the V rows (lane l of
  // piece c writes chunk 64 c + l of the slot and fetches the logical chunk the swizzle
  // puts there); rows past N read as zeros --------------------------------------------------
  uint32_t cvoff[PPW];
#pragma unroll
  for (int cc = 0; cc < PPW; ++cc) {
    const int f = (wid + NW * cc) * 64 + lane, row = f / CPR, ph = f % CPR;
    cvoff[cc] = (uint32_t)(row * D + (ph ^ swz_b<D>(row)) * 8) * 2u;
  }
  const uint32_t k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(kring + wid * 64));
  const uint32_t v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(vring + wid * 64));
  auto copy = [&](int g, int sl, int cc) __attribute__((always_inline)) {
    const int row0 = g * KB;
    const uint32_t nbytes = sclamp(N - row0, KB) * (uint32_t)(D * 2);
    const int piece = cc % PPW;
    const bool is_k = cc < PPW;
    const uint16_t* src = (is_k ? p.k : p.v) + head + (size_t)row0 * D;
    lds_copy16(buffer_rsrc((uint64_t)(uintptr_t)src, nbytes), cvoff[piece], is_k ? k_lds : v_lds,
               sl * SLOT * 16 + piece * NW * 1024);
  };

  // ---- per-lane LDS read addresses (ring base included, held opaque) -----------------
  uint32_t raddr[2][NDS];  // rows: [w: K, V][ds]
  {
    const int row = key_of_row(l32);
    const uint32_t r = (uint32_t)((row * CPR + (hh ^ swz_b<D>(row))) * 16);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      raddr[0][ds] = (uint32_t)(uintptr_t)kring + (r ^ (uint32_t)(ds << 5));
      raddr[1][ds] = (uint32_t)(uintptr_t)vring + (r ^ (uint32_t)(ds << 5));
      asm volatile("" : "+v"(raddr[0][ds]), "+v"(raddr[1][ds]));
    }
  }
  uint32_t taddr[NDB][2];  // transposed K: [db][h]
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      taddr[db][h] = (uint32_t)(uintptr_t)kring + bwd_tr_off<D>(lane, db, h);
      asm volatile("" : "+v"(taddr[db][h]));
    }
  typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
  // the A operand of operand slot s of an iteration: s < NA, dQ step s (16-key half
  // s / NDB, head dims 32 (s % NDB) ..) from K^T of slot slt; s >= NA, the K (even) or V
  // (odd) rows of head-dim step (s - NA) / 2 of slot slr
  auto operand = [&](int s, int slt, int slr) __attribute__((always_inline)) {
    if (s < NA) {
      const uint32_t off = (uint32_t)(slt * SLOT * 16 + (s / NDB) * 16 * CPR * 16);
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(uintptr_t)(taddr[s % NDB][0] + off));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(uintptr_t)(taddr[s % NDB][1] + off));
      const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
      return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
    }
    const int w = (s - NA) % 2, ds = (s - NA) / 2;
    return *(lds_u32x4_t*)(uintptr_t)(raddr[w][ds] + (uint32_t)(slr * SLOT * 16));
  };

  // ---- the softmax terms of one key block ------------------------------------------------
  typedef f32x16_t Tiles[NQB];
  typedef u32x4_t DsOps[NQB][2];
  constexpr DqOpSched OPS = kDqOps<PS, NC, NA, NOP, NQB>;
  float xq[2][2], dq3[3][2], pq[2][2], eq[2][2];
  auto soft_op = [&](const Tiles& s, const Tiles& dp, DsOps& dsop, int o)
      __attribute__((always_inline)) {
    const int v = OPS.code[o] / 10, op = OPS.code[o] % 10;
    const int qb = v / 8, r0 = 2 * (v % 8);
    if (op < 2) {
      xq[v % 2][op] = __builtin_fmaf(s[qb][r0 + op], c, -L2[qb]);
      asm volatile("" : "+v"(xq[v % 2][op]));
    } else if (op < 4) {
      pq[v % 2][op - 2] = __builtin_amdgcn_exp2f(xq[v % 2][op - 2]);
      asm volatile("" : "+v"(pq[v % 2][op - 2]));
    } else if (op < 6) {
      dq3[v % 3][op - 4] = dp[qb][r0 + op - 4] - Dq[qb];
      asm volatile("" : "+v"(dq3[v % 3][op - 4]));
    } else if (op < 8) {
      eq[v % 2][op - 6] = pq[v % 2][op - 6] * dq3[v % 3][op - 6];
      asm volatile("" : "+v"(eq[v % 2][op - 6]));
    } else {
      uint32_t w = E::pack(eq[v % 2][0], eq[v % 2][1]);
      asm volatile("" : "+v"(w));
      dsop[qb][r0 / 8][(r0 % 8) / 2] = w;
    }
  };
  // causal: register r (key 32 g + 8 hh + key_of_reg(r, 0)) keeps when that key <= the
  // lane's query; only blocks that reach past the query block's first query need it
  auto mask = [&](Tiles& s, int g) __attribute__((always_inline)) {
    if (!CAUSAL) return;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (g * KB + KB - 1 <= qbase[qb]) continue;
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[qb]));
      const int t = qi[qb] - (g * KB + 8 * hh);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[qb][r];
        asm("v_cmp_le_i32 vcc, %2, %1\n\tv_cndmask_b32 %0, %3, %0, vcc"
            : "+v"(x) : "v"(t), "n"(key_of_reg(r, 0)), "v"(s_mask) : "vcc");
        s[qb][r] = x;
      }
    }
  };
  auto zero = [](Tiles& x) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[qb][r] = 0.f;
  };

  // ---- one iteration: dQ of block t; softmax terms of block t+1; S, dP of block t+2 ----
  u32x4_t onext[PS];  // operands of the next iteration's first PS operand slots
  auto iteration = [&](int u, int t, Tiles& s_new, Tiles& dp_new, const Tiles& s_mid,
                       const Tiles& dp_mid, DsOps& ds_mid, const DsOps& ds_cur)
      __attribute__((always_inline)) {
    const int sl0 = u, sl1 = (u + 1) % R, sl2 = (u + 2) % R, slc = (u + AHEAD) % R;
    u32x4_t opd[NOP];
#pragma unroll
    for (int s = 0; s < PS; ++s) opd[s] = onext[s];
    zero(s_new);
    zero(dp_new);
#pragma unroll
    for (int sl = 0; sl < NOP * NQB; ++sl) {
      const int s = sl / NQB, qb = sl % NQB;
      // one LDS wait per two operand slots: the operands of s and s + 1 together
      if (qb == 0 && s % 2 == 0) {
        asm volatile("" ::"v"(opd[s]), "v"(opd[s + 1]));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (s < NA) {
        // keep the previous product's sources live until this one (the inline-assembly
        // MFMAs read them over several cycles)
        if (sl > 0) {
          const int ps = (sl - 1) / NQB, pq2 = (sl - 1) % NQB;
          asm volatile("" ::"v"(opd[ps]), "v"(ds_cur[pq2][ps / NDB]));
        }
        mfma_acc_agpr<BF16>(dq[qb][s % NDB], opd[s], ds_cur[qb][s / NDB]);
      } else if ((s - NA) % 2 == 0) {
        s_new[qb] = E::mfma(opd[s], qf[qb][(s - NA) / 2], s_new[qb]);
      } else {
        dp_new[qb] = E::mfma(opd[s], dof[qb][(s - NA) / 2], dp_new[qb]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (qb == 0) {
        if (s + PS < NOP) opd[s + PS] = operand(s + PS, sl0, sl2);
        else onext[s + PS - NOP] = operand(s + PS - NOP, sl1, sl1);
        if (s < NA && s % 2 == 1 && s / 2 < NC) copy(t + AHEAD, slc, s / 2);
      }
#pragma unroll
      for (int o = OPS.first[sl]; o < OPS.first[sl + 1]; ++o) soft_op(s_mid, dp_mid, ds_mid, o);
      __builtin_amdgcn_sched_barrier(0);
      if (sl == NA * NQB - 1) asm volatile("" ::"v"(opd[NA - 1]), "v"(ds_cur[NQB - 1][1]));
    }
    mask(s_new, t + 2);
  };

  // ---- prologue: blocks 0 .. 4 copied; S, dP of block 0, its softmax terms; S, dP of
  // block 1 ---------------------------------------------------------------------------------
#pragma unroll
  for (int b = 0; b < AHEAD; ++b)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) copy(b, b, cc);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((AHEAD - 2) * NC) : "memory");  // blocks 0, 1
  __syncthreads();
  Tiles sA, sB, dA, dB;
  DsOps dsA, dsB;
  zero(sA);
  zero(dA);
  zero(sB);
  zero(dB);
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    const u32x4_t ka = operand(NA + 2 * ds, 0, 0), va = operand(NA + 1 + 2 * ds, 0, 0);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      sA[qb] = E::mfma(ka, qf[qb][ds], sA[qb]);
      dA[qb] = E::mfma(va, dof[qb][ds], dA[qb]);
    }
  }
  mask(sA, 0);
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    const u32x4_t kb = operand(NA + 2 * ds, 0, 1), vb = operand(NA + 1 + 2 * ds, 0, 1);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      sB[qb] = E::mfma(kb, qf[qb][ds], sB[qb]);
      dB[qb] = E::mfma(vb, dof[qb][ds], dB[qb]);
    }
  }
#pragma unroll
  for (int o = 0; o < OPS.n; ++o) soft_op(sA, dA, dsA, o);
  mask(sB, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // blocks 2 .. 4
  __syncthreads();
#pragma unroll
  for (int s = 0; s < PS; ++s) onext[s] = operand(s, 0, 0);

  // ---- main loop, unrolled over the ring (S/dP tiles and dS operands alternate between
  // the even (A) and odd (B) buffers) ------------------------------------------------------
  for (int t0 = 0; t0 < nb; t0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int t = t0 + u;
      if (t >= nb) break;
      if (u % 2 == 0) iteration(u, t, sA, dA, sB, dB, dsB, dsA);
      else iteration(u, t, sB, dB, sA, dA, dsA, dsB);
      // every copy but this iteration's has landed; the barrier follows this wave's last
      // read of block t's slot (its PS reads of block t+1's K^T may stay in flight)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NC) : "memory");
      asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(2 * PS) : "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(dq[qb][db]));
    if (qi[qb] < N) bwd_store_rows<BF16, D>(p.dq + head, dq[qb], qi[qb], hh, p.scale);
  }
}

}  // namespace fa
