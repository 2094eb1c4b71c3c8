// fa_fwd_wide.hpp — FA2-order attention forward for gfx950 (MI355X): one wave per
// SIMD, 64 queries per wave, for head dims 64 and 128.
//
// Algorithm ([P1] currybab.bearblog.dev, "Triton으로 FlashAttention 구현하기 전에 -
// FA1, 2 forward pass", section "FlashAttention 2 forward pass 알고리즘 분석"): the
// query row block is the outer loop (one workgroup per query block, head and batch),
// key/value blocks stream through LDS in the inner loop, each row keeps its running
// max and sum on chip, rescales the unnormalised output by alpha = exp(m_old - m_new)
// only, and divides once at the end. Waves own disjoint query rows (split-Q), so no
// cross-wave merge exists.
//
// Why a second fast kernel: with 32 queries per wave, every K or V operand read from
// LDS feeds exactly one 32x32x16 MFMA, and the LDS read bandwidth of a CU then equals
// its MFMA rate, so LDS and the matrix cores bound each other. Here each wave owns
// two 32-query column blocks and every operand read from LDS feeds two MFMAs, which
// halves the LDS traffic per flop. The price is registers: the two output
// accumulators alone take 128 of them at d = 128, so a wave gets the whole register
// file of its SIMD (one wave per SIMD, four per workgroup) and hides latency by
// software pipelining only.
//
// gfx950 mapping:
//   * K and V tiles are copied HBM -> LDS by buffer_load_dwordx4 ... lds (no register
//     staging) into a ring of R slots each. Iteration j issues K_{j+R} and V_{j+R-1};
//     every copy has R - 1 iterations to land, and the end-of-iteration wait leaves
//     the newest R - 2 iterations of copies in flight (vmcnt counts this wave's copies
//     in issue order). One barrier per iteration makes the other waves' copies
//     visible and frees the slots for the next copies.
//   * K runs one tile ahead of V: while tile j is finished, the S^T MFMAs of tile j+1
//     are interleaved with the first half of the exponentials of tile j, and the P V
//     MFMAs of tile j with the second half and then with the row max of tile j+1.
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}; each lane owns
//     one query column per block, so the running max/sum and the alpha rescale are
//     in-lane, and the S^T accumulator rounded to 16 bits is the B operand of P V
//     (key rows enter with bits 2 and 3 of the row index swapped).
//   * LDS layout, XOR swizzles, transposed V reads (ds_read_b64_tr_b16), exp2 with the
//     log2(e) factor folded into the scale, the lazy rescale threshold tau and the
//     causal tile skipping are those of the 32-query kernel.
#pragma once

#include "fa_common.hpp"

#ifndef FA_W_PF
#define FA_W_PF 2         // MFMA steps an LDS operand read runs ahead
#endif
#ifndef FA_W_KPRE
#define FA_W_KPRE 1       // first K operands of a tile read at the end of the previous one
#endif
#ifndef FA_W_PAIRS_B128
#define FA_W_PAIRS_B128 19  // score pairs (of 32) exponentiated in the S^T block, d = 128
#endif
#ifndef FA_W_PAIRS_B64
#define FA_W_PAIRS_B64 18   // the same for d = 64
#endif
#define FA_W_PAIRS_B(D) ((D) == 128 ? FA_W_PAIRS_B128 : FA_W_PAIRS_B64)

namespace fa {

template <int D_, int BC_, int R_>
struct WideGeom {
  static constexpr int D = D_;
  static constexpr int BC = BC_;
  static constexpr int R = R_;                   // ring slots per tensor
  static constexpr int NW = 4;                   // waves per workgroup, one per SIMD
  static constexpr int QB = 2;                   // 32-query blocks per wave
  static constexpr int BR = NW * QB * 32;        // queries per workgroup
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int CHUNKS = BC * CPR;        // chunks per K (or V) tile
  static constexpr int INSTR = CHUNKS / 64;      // 1 KB wave copies per tile and tensor
  static constexpr int PER_WAVE = INSTR / NW;    // copies per wave per tile and tensor
  static constexpr int NQK = (BC / 32) * (D / 16);  // S^T steps per tile (2 MFMAs each)
  static constexpr int NPV = (D / 32) * (BC / 16);  // P V steps per tile (2 MFMAs each)
  static constexpr int NST = BC / 16;            // 16-key P operands per query block
  static_assert(D == 64 || D == 128, "fast path head dims");
  static_assert(BC % 32 == 0 && CHUNKS % 64 == 0, "whole MFMA blocks and wave copies");
  static_assert(INSTR % NW == 0 && PER_WAVE >= 1, "every wave issues the same copies");
  static_assert(2 * PER_WAVE <= NQK, "copies fit in the S^T pipeline steps");
  static_assert(R >= 2 && R % 2 == 0, "ring of an even number of slots");
  static_assert(2 * PER_WAVE * (R - 1) <= 63, "outstanding copies fit the vmcnt field");
};

// Checks the softmax schedule of the P V block: with the units of pairs ub/3 .. npair-1
// spread evenly over `ces` slots, the last unit of every pair lands at least one slot
// before the first MFMA that reads its P step (pairs npair/nst per step, steps of `db`
// slot pairs).
constexpr bool fa_wide_exp_deadlines(int npair, int nst, int db, int ub, int ces) {
  const int uc = 3 * npair - ub;
  if (uc == 0) return true;
  if (ces <= 0 || ub % 3 != 0) return false;
  for (int v = ub / 3; v < npair; ++v) {
    const int rel = 3 * v + 2 - ub;
    int slot = 0;
    while ((slot + 1) * uc / ces <= rel) ++slot;  // slot s holds units [s uc/ces, (s+1) uc/ces)
    if (slot > 2 * (v / (npair / nst)) * db - 2) return false;
  }
  return true;
}

// O~ += A B with the accumulator held in AGPRs (the S^T accumulators stay in VGPRs,
// where the VALU reads them). Written out because the compiler picks one register
// file for all MFMA accumulators of a kernel.
template <bool BF16>
__device__ __forceinline__ void mfma_acc_agpr(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  if (BF16)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Raw buffer resource over `bytes` bytes at address a (stride 0, 32-bit format): reads
// past the end return zeros.
__device__ __forceinline__ u32x4_t buffer_rsrc(uint64_t a, uint32_t bytes) {
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kBufferWord3};
}

// The copies and the Q loads are issued as inline assembly, so the compiler's memory
// counter model does not see them and adds no waits of its own: the kernel orders
// them with explicit vmcnt waits and its ring barrier. One 16-byte-per-lane HBM -> LDS
// copy: lane l's 16 bytes at byte offset voff of the buffer land at LDS address
// lds + lds_off + 16 l (M0 holds the wave's LDS base); bytes past the buffer's size
// read as 0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(u32x4_t rsrc, uint32_t voff, uint32_t lds,
                                           int lds_off /* a constant after unrolling */) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds), "n"(lds_off) : "m0", "scc");
}
#pragma clang diagnostic pop
// 16-byte global load; the result may only be read after an explicit vmcnt wait
// that covers it.
__device__ __forceinline__ u32x4_t global_load16(const uint16_t* p) {
  u32x4_t x;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x) : "v"(p));
  return x;
}

// x = (c <= t) ? x : -inf, with c a constant after unrolling. Compare and select
// stay one pair, so no lane masks pile up in scalar registers across a tile.
__device__ __forceinline__ float keep_if_le(float x, int c, int t) {
  // v_cndmask reads VCC, so -inf comes from a register (one constant-bus operand)
  asm("v_cmp_le_i32 vcc, %2, %1\n\tv_cndmask_b32 %0, %3, %0, vcc"
      : "+v"(x) : "v"(t), "n"(c), "v"(-__builtin_inff()) : "vcc");
  return x;
}

template <bool BF16, int D, bool CAUSAL, int BC, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fa_fwd_wide_kernel(const Params p) {
  using G = WideGeom<D, BC, R>;
  using E = Elt<BF16>;
  constexpr int NW = G::NW, CPR = G::CPR, NQK = G::NQK, NPV = G::NPV, NST = G::NST;
  constexpr int CHUNKS = G::CHUNKS, PW = G::PER_WAVE, NDMA = 2 * PW;
  // ---- pipeline schedule -----------------------------------------------------------
  // Each tile runs as two blocks of MFMA slots: the S^T MFMAs of the next tile (block
  // B), then the P V MFMAs of this tile (block C). A slot issues one MFMA and then a
  // batch of other instructions (LDS operand reads, copies, softmax work) that the wave
  // issues while the matrix core executes it; slots are fenced from each other, so two
  // MFMAs are never issued back to back (the second would stall the wave for the whole
  // first one) and the VALU work is spread evenly over the tile.
  //
  // A lane holds NPAIR pairs of scores per tile (both query blocks). The softmax work
  // of pair v is three units: the two exponentials, then the accumulation into the
  // running sums and the 16-bit packing of the P operand. The first PAIRS_B pairs are
  // done in block B, the rest in block C, each at least one slot before the first P V
  // MFMA that reads them. Block C also carries the row max of the next tile (one max3
  // per pair) and, after it, the rescale vote.
  constexpr int SB_N = 2 * NQK;                 // slots of block B
  constexpr int SC_N = 2 * NPV;                 // slots of block C
  constexpr int NPAIR = BC / 2;                 // score pairs per lane and tile
  constexpr int PAIRS_B = FA_W_PAIRS_B(D) < NPAIR ? FA_W_PAIRS_B(D) : NPAIR;
  constexpr int UB = 3 * PAIRS_B;               // softmax units in block B
  constexpr int UC = 3 * NPAIR - UB;            // softmax units in block C
  // block C carries them up to two slots before the first MFMA of the last P step
  constexpr int C_EXP_SLOTS = 2 * (NST - 1) * (D / 32) - 1;
  constexpr int M_SLOTS = SC_N - 3;             // max units; the vote is in the next slot
  static_assert(PAIRS_B >= NPAIR / NST, "the first P step is complete before block C");
  static_assert(fa_wide_exp_deadlines(NPAIR, NST, D / 32, UB, C_EXP_SLOTS),
                "every P operand is complete one slot before the MFMA that reads it");
  // K ring and V ring; slot u of a ring holds one tile at offset u * CHUNKS
  __shared__ __attribute__((aligned(1024))) u32x4_t kbuf[R * CHUNKS];
  __shared__ __attribute__((aligned(1024))) u32x4_t vbuf[R * CHUNKS];
  // landing area of the L2-warming copies below (their data is never read)
  __shared__ __attribute__((aligned(1024))) u32x4_t warm[NW * 64];

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
  // The workgroup's 256 queries are eight 32-query blocks; wave w owns blocks w and 7 - w
  // (query block qb = 0, 1 of the wave), so under the causal mask the four waves end
  // their rows within one key tile of each other.
  const int qbase[2] = {q0 + 32 * wid, q0 + 32 * (2 * NW - 1 - wid)};
  const int wq0 = qbase[0];  // the wave's first query
  const int q_end = min(q0 + G::BR, N);
  const int n_kt = CAUSAL ? (q_end + BC - 1) / BC : (N + BC - 1) / BC;
  const bool wave_live = wq0 < N;
  const int w_last_q = min(qbase[1] + 32, N) - 1;
  const int w_kt = CAUSAL ? min(n_kt, w_last_q / BC + 1) : n_kt;

  // ---- HBM -> LDS copies ---------------------------------------------------------
  // Lane `lane` of copy instruction i writes LDS chunk 64 i + lane = (row, physical
  // chunk) of a tile; it fetches the logical chunk that the swizzle puts there.
  // Copy ii covers rows 64 NW ii / CPR further down than copy 0, a multiple of 16 rows,
  // and both swizzles depend on the row only modulo 16: the byte offsets of copy ii
  // are those of copy 0 plus II_BYTES * ii.
  constexpr uint32_t II_BYTES = NW * 64 * 16;
  static_assert((NW * 64 / CPR) % 16 == 0, "copies are whole 16-row groups");
  uint32_t koff, voff;
  {
    const int f = wid * 64 + lane, row = f / CPR, ph = f % CPR;
    koff = (uint32_t)(row * D + (ph ^ swz_k<D>(row)) * 8) * 2u;
    voff = (uint32_t)(row * D + (ph ^ swz_v<D>(row)) * 8) * 2u;
  }
  // One copy of tile j. The buffer resource spans the tile's rows below N, so chunks
  // of rows past N read as zeros (their scores are masked to -inf). Tiles past the
  // last are clamped to it: such a copy lands in a slot no later tile reads.
  // The buffer of tile j spans its rows below N: the range check zero-fills the rest.
  auto tile_rsrc = [&](const uint16_t* src, int j) {
    const int k0 = min(j, n_kt - 1) * BC;
    return buffer_rsrc((uint64_t)(uintptr_t)(src + (size_t)k0 * D),
                       (uint32_t)(min(N - k0, BC) * D * 2));
  };
  // LDS byte address of this wave's first chunk in slot 0 of each ring; the slot
  // and copy offsets are immediates
  const uint32_t k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(kbuf + wid * 64));
  const uint32_t v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(vbuf + wid * 64));
  struct Copies {
    int k_slot, v_slot;
    int jk, jv;
  };
  // copy step i of a tile: K copies first, then V copies
  auto copy_step = [&](const Copies& cp, int i) {
    if (i < PW)
      lds_copy16(tile_rsrc(kg, cp.jk), koff + II_BYTES * i, k_lds,
                 cp.k_slot * CHUNKS * 16 + i * NW * 1024);
    else if (i < NDMA)
      lds_copy16(tile_rsrc(vg, cp.jv), voff + II_BYTES * (i - PW), v_lds,
                 cp.v_slot * CHUNKS * 16 + (i - PW) * NW * 1024);
  };
  auto copy_all = [&](const Copies& cp) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) copy_step(cp, i);
  };

  // ---- Q fragments (B operands of S^T = K Q^T), in registers for the whole loop -----
  // Issued before any copy, so the first wait for K_0 also covers them. Rows past N
  // load row N-1: their columns are never stored.
  u32x4_t qf[2][D / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = min(qbase[qb] + l32, N - 1);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      qf[qb][ds] = global_load16(qg + (size_t)qi * D + ds * 16 + hh * 8);
  }

  // ---- prologue copies: K_0, then (K_t, V_{t-1}) for t = 1 .. R-1 ---------------------
  // the same (K, V) pairing as the main loop, so one vmcnt formula serves both
#pragma unroll
  for (int i = 0; i < PW; ++i) copy_step(Copies{0, 0, 0, 0}, i);
#pragma unroll
  for (int t = 1; t < R; ++t) copy_all(Copies{t, t - 1, t, t - 1});

  // ---- running state ---------------------------------------------------------------
  f32x16_t oacc[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  float ms[2] = {0.f, 0.f};
  float ls[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // per-lane running sums, two chains each
  const float c = p.c;

  // ---- per-lane LDS read addresses (see the 32-query kernel for the bank analysis) --
  // Absolute LDS byte addresses of slot 0, pinned in registers, so that the slot and
  // step offsets (all below 64 KB) become the immediate offsets of the reads even
  // when the ring itself lies above 64 KB.
  // K: the row pitch is a multiple of 128 bytes and the swizzle acts on chunk bits
  // only, so the address of step ds is that of step 0 with (2 ds) << 4 XORed in
  // (the logical chunk 2 ds + hh enters the XOR linearly).
  uint32_t kaddr0;
  {
    const int row = key_of_row(l32);
    kaddr0 = (uint32_t)(uintptr_t)kbuf + (row * CPR + (hh ^ swz_k<D>(row))) * 16;
    asm volatile("" : "+v"(kaddr0));
  }
  uint32_t vaddr[D / 32];
  {
    const int g16 = lane >> 4, t4 = (lane & 15) >> 2, u4 = lane & 3;
    const int row = (g16 >> 1) * 8 + t4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      vaddr[db] = (uint32_t)(uintptr_t)vbuf +
                  (row * CPR + ((4 * db + 2 * (g16 & 1) + (u4 >> 1)) ^ swz_v<D>(row))) * 16 +
                  (u4 & 1) * 8;
      asm volatile("" : "+v"(vaddr[db]));
    }
  }
  typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
  auto k_frag = [&](int slot, int i) {
    const int kb = i % (BC / 32), ds = i / (BC / 32);
    return *(lds_u32x4_t*)(uintptr_t)((kaddr0 ^ (uint32_t)(ds << 5)) + slot * CHUNKS * 16 +
                                      kb * 32 * CPR * 16);
  };
  // half h (keys 4h .. 4h+3 of each 8-key group) of the V^T operand of P V step i
  auto v_half = [&](int slot, int i, int h) {
    const int db = i % (D / 32), st = i / (D / 32);
    const uint32_t b = vaddr[db] + slot * CHUNKS * 16;
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (lds_s16x4_t*)(uintptr_t)(b + (16 * st + 4 * h) * CPR * 16)));
  };

  // S^T accumulators of one key tile: [key block][query block]; score e of a lane's
  // query column (0 <= e < BC/2) is register e % 16 of key block e / 16
  typedef f32x16_t STile[BC / 32][2];
  auto zero = [](STile& s) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
  };
  // S^T of a whole tile from K slot kst, without interleaved work
  auto qk_plain = [&](int kst, STile& s) {
    zero(s);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int kb = i % (BC / 32), ds = i / (BC / 32);
      const u32x4_t kf = k_frag(kst, i);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = E::mfma(kf, qf[qb][ds], s[kb][qb]);
    }
  };

  // -inf on keys past N and, under the causal mask, on keys after the query; only
  // tiles that reach past N or cross the diagonal need it
  auto mask = [&](STile& s, int j) {
    const int k0 = j * BC;
    const bool masked = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > wq0);
    if (!masked) return;
    // With key = k0 + 8 hh + c (c = 32 kb + key_of_reg(r, 0), a constant per register),
    // a score is kept iff c <= t, where t is the last allowed key of the lane's query
    // (below N, and not after the query under the causal mask) minus k0 + 8 hh: one
    // compare against a per-lane value per register.
    const int base = k0 + 8 * hh;
    // the compares are inline assembly, which the compiler's hazard tracking does
    // not see: wait out the S^T MFMAs first (an 8-pass XDL result needs about a
    // dozen wait states before a VALU access), taking the tile as operands so the
    // compares stay behind the padding
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0][0]));
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        if (kb + qb > 0) asm volatile("" : "+v"(s[kb][qb]));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int last = CAUSAL ? min(N - 1, qbase[qb] + l32) : N - 1;
      const int t = last - base;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][qb][r] = keep_if_le(s[kb][qb][r], kb * 32 + key_of_reg(r, 0), t);
    }
  };

  // m_new = max(m_old, rowmax S); alpha = exp2(m_old - m_new) rescales l and O~ of one
  // query block. The wave skips it when no row's max rose by more than tau (log2 units).
  // The compiler does not know that the P V MFMAs (inline assembly) write O~, so it
  // inserts no wait states before VALU accesses of O~: this pads them (an 8-pass
  // XDL result needs about a dozen) and, by taking the accumulators as operands,
  // keeps every such access after the padding.
  auto drain_o = [&](int qb) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(oacc[0][qb]));
#pragma unroll
    for (int db = 1; db < D / 32; ++db) asm volatile("" : "+a"(oacc[db][qb]));
  };
  auto grow_max = [&](int qb, float mxs, uint64_t need) {
    if (need != 0) {
      const float ms_new = __builtin_fmaxf(ms[qb], mxs);
      const float alpha = __builtin_amdgcn_exp2f(ms[qb] - ms_new);
      ms[qb] = ms_new;
      ls[qb][0] *= alpha;
      ls[qb][1] *= alpha;
      drain_o(qb);
      // one 16-register block at a time (it passes through VGPRs), so the rescale
      // needs few registers while both S^T tiles are live
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
        asm volatile("" : "+a"(oacc[db][qb]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  u32x4_t pb[2][NST];  // P~ of the current tile, packed as P V operands

  // Softmax unit u of the current tile (pair v = u / 3): units 3v and 3v+1 are the two
  // exponentials of the pair, unit 3v+2 adds them to the running sums and packs them
  // into the P operand. Pair v is scores e, e+1 (e = 8 (v / 8) + 2 (v % 4)) of query
  // block (v / 4) % 2, i.e. the P operands are produced in the order the P V steps
  // consume them (16-key step major, query block minor). Results are pinned, so each
  // unit is computed in the slot that issues it.
  float pe[2];  // the exponentials of the pair in flight
  auto exp_unit = [&](const STile& s, int u) {
    const int v = u / 3, k = u % 3, qb = (v / 4) % 2, e = 8 * (v / 8) + 2 * (v % 4);
    if (k < 2) {
      // c > 0 on this path, so a masked score (-inf) gives exp2(-inf) = 0 exactly
      pe[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[(e + k) / 16][qb][(e + k) % 16], c, -ms[qb]));
      asm volatile("" : "+v"(pe[k]));
    } else {
      ls[qb][0] += pe[0];
      ls[qb][1] += pe[1];
      uint32_t w = E::pack(pe[0], pe[1]);
      asm volatile("" : "+v"(w), "+v"(ls[qb][0]), "+v"(ls[qb][1]));
      pb[qb][e / 8][(e % 8) / 2] = w;
    }
  };
  // Row max unit w of the next tile: one max3 over a pair of its scores, into one of two
  // chains per query block.
  auto max_unit = [&](const STile& s, float (&m)[2][2], int w) {
    const int qb = w / (NPAIR / 2), k = w % (NPAIR / 2), e = 2 * k;
    m[qb][k % 2] = __builtin_fmaxf(m[qb][k % 2], __builtin_fmaxf(s[e / 16][qb][e % 16],
                                                                   s[e / 16][qb][(e + 1) % 16]));
    asm volatile("" : "+v"(m[qb][k % 2]));
  };

  // Block B: S^T of tile j+1, slot 2i + qb = step i (key block i % (BC/32), head-dim
  // slice i / (BC/32)) for query block qb. Besides its share of the softmax units of tile
  // j, a slot carries the K operand read for FA_W_PF steps later (after the first MFMA
  // of a step), this wave's copies of later tiles (one every SB_N / NDMA slots, so the
  // four waves do not queue their copies at once) and, in the last steps, the first V^T
  // operand reads of block C.
  static_assert(SB_N % NDMA == 0, "copies spread evenly over block B");
  u32x4_t kpre[FA_W_PF];  // the first K operands of the next block B
  auto block_b = [&](int k_next, STile& s_next, const STile& s_cur, const Copies& cp,
                     int v_cur, u32x2_t (&vpre)[FA_W_PF][2]) {
    zero(s_next);
    u32x4_t kf[NQK];
#pragma unroll
    for (int i = 0; i < FA_W_PF; ++i) kf[i] = FA_W_KPRE ? kpre[i] : k_frag(k_next, i);
#pragma unroll
    for (int sl = 0; sl < SB_N; ++sl) {
      const int i = sl / 2, qb = sl % 2, kb = i % (BC / 32), ds = i / (BC / 32);
      s_next[kb][qb] = E::mfma(kf[i], qf[qb][ds], s_next[kb][qb]);
      __builtin_amdgcn_sched_barrier(0);
      if (qb == 0 && i + FA_W_PF < NQK) kf[i + FA_W_PF] = k_frag(k_next, i + FA_W_PF);
      if (sl % (SB_N / NDMA) == 1) copy_step(cp, sl / (SB_N / NDMA));
      if (i >= NQK - FA_W_PF) vpre[i - (NQK - FA_W_PF)][qb] = v_half(v_cur, i - (NQK - FA_W_PF), qb);
#pragma unroll
      for (int u = sl * UB / SB_N; u < (sl + 1) * UB / SB_N; ++u) exp_unit(s_cur, u);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Block C: P V of tile j, slot 2i + qb = step i (head-dim block i % (D/32), P step
  // i / (D/32)) for query block qb. A slot carries one half of the V^T operand read for
  // FA_W_PF steps later, the remaining softmax units of tile j (up to two slots before
  // their P step is read), the row max of tile j+1 and, in slot M_SLOTS, the exchange
  // of the maxima between the two wave halves and the wave's rescale votes. Returns the
  // row maxima of the two query blocks of tile j+1 (log2 units) and the votes.
  // The last slots, which read no V^T operands, read the first K operands of the next
  // tile's block B (K slot k_after), so that block starts without an LDS wait.
  static_assert(2 * (NPV - FA_W_PF) + 2 * FA_W_PF <= SC_N, "slots for the K look-ahead");
  auto block_c = [&](int v_cur, int k_after, const STile& s_cur, const STile& s_next,
                     const u32x2_t (&vpre)[FA_W_PF][2], float& mx0, float& mx1, uint64_t& need0,
                     uint64_t& need1) {
    float m[2][2] = {{-__builtin_inff(), -__builtin_inff()},
                     {-__builtin_inff(), -__builtin_inff()}};
    u32x2_t vh[NPV][2];
#pragma unroll
    for (int i = 0; i < FA_W_PF; ++i) {
      vh[i][0] = vpre[i][0];
      vh[i][1] = vpre[i][1];
    }
#pragma unroll
    for (int sl = 0; sl < SC_N; ++sl) {
      const int i = sl / 2, qb = sl % 2, db = i % (D / 32), st = i / (D / 32);
      // The compiler does not know the MFMAs below read their sources over several
      // cycles (they are inline assembly): keep the previous step's sources live
      // until this step, so no result is written into them right behind the MFMA.
      if (qb == 0 && i > 0)
        asm volatile("" ::"v"(vh[i - 1][0]), "v"(vh[i - 1][1]), "v"(pb[0][(i - 1) / (D / 32)]),
                     "v"(pb[1][(i - 1) / (D / 32)]));
      const u32x4_t vf = {vh[i][0][0], vh[i][0][1], vh[i][1][0], vh[i][1][1]};
      mfma_acc_agpr<BF16>(oacc[db][qb], vf, pb[qb][st]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + FA_W_PF < NPV) vh[i + FA_W_PF][qb] = v_half(v_cur, i + FA_W_PF, qb);
      if (FA_W_KPRE && qb == 0 && i >= NPV - FA_W_PF) kpre[i - (NPV - FA_W_PF)] = k_frag(k_after, i - (NPV - FA_W_PF));
      if (sl < C_EXP_SLOTS) {
#pragma unroll
        for (int u = sl * UC / C_EXP_SLOTS; u < (sl + 1) * UC / C_EXP_SLOTS; ++u)
          exp_unit(s_cur, UB + u);
      }
      if (sl < M_SLOTS) {
#pragma unroll
        for (int w = sl * NPAIR / M_SLOTS; w < (sl + 1) * NPAIR / M_SLOTS; ++w)
          max_unit(s_next, m, w);
      }
      if (sl == M_SLOTS) {
        mx0 = xhalf_max(__builtin_fmaxf(m[0][0], m[0][1])) * c;
        mx1 = xhalf_max(__builtin_fmaxf(m[1][0], m[1][1])) * c;
        need0 = __builtin_amdgcn_ballot_w64(mx0 > ms[0] + p.tau);
        need1 = __builtin_amdgcn_ballot_w64(mx1 > ms[1] + p.tau);
        asm volatile("" : "+v"(mx0), "+v"(mx1), "+s"(need0), "+s"(need1));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One key tile j whose masked S^T is in s_cur and whose max is already folded into
  // ms: exponentials and P V of tile j, overlapped with the S^T, mask and max of tile
  // j+1 (from K slot k_next). On a wave's last tile the look-ahead reads a slot that
  // holds a stale or clamped tile, and its result is dropped (`next` false).
  auto tile = [&](const STile& s_cur, STile& s_next, int k_next, int v_cur, int k_after, int j,
                  bool next, const Copies& cp) {
    u32x2_t vpre[FA_W_PF][2];
    block_b(k_next, s_next, s_cur, cp, v_cur, vpre);
    mask(s_next, j + 1);
    float mx0, mx1;
    uint64_t need0, need1;
    block_c(v_cur, k_after, s_cur, s_next, vpre, mx0, mx1, need0, need1);
    if (next) {
      grow_max(0, mx0, need0);
      grow_max(1, mx1, need1);
    }
  };

  // After this wave's copies for tiles up to (K_{j+2}, V_{j+1}) have landed (and
  // K_{j+3}, whose first operands the next tile reads ahead), the newest RING_LAG
  // iterations of copies may still be in flight.
  constexpr int RING_LAG = FA_W_KPRE ? R - 3 : R - 2;
  static_assert(RING_LAG >= 0, "ring deep enough for the K look-ahead");
  auto wait_ring = [&]() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA * RING_LAG) : "memory");
  };
  // Workgroup barrier for the ring. This wave's LDS reads are complete before it
  // (lgkmcnt), so after it another wave may overwrite the slots they read; copies
  // are ordered by the explicit vmcnt waits. The memory clobber keeps LDS accesses
  // and copies on their side of it. (A full __syncthreads fence would also wait for
  // the copies still in flight, which the ring is there to avoid.)
  auto ring_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // ---- S^T of tile 0 and the initial reference max ------------------------------------
  STile sa, sb;
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA * (R - 1)) : "memory");  // Q and K_0
  // Q has landed: sign flip for a negative scale, then Q lives in AGPRs (MFMA source
  // operands may come from either register file), leaving the VGPRs to the S^T
  // tiles and the VALU work
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      asm volatile("" : "+v"(qf[qb][ds]));
      qf[qb][ds] ^= p.qsign;
      asm volatile("" : "+a"(qf[qb][ds]));
    }
  ring_barrier();
  if (wave_live) {
    qk_plain(0, sa);
    mask(sa, 0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sa[kb][qb][r]);
      // tile 0 holds key 0, allowed for every row: finite
      ms[qb] = xhalf_max(mx) * c;
    }
  }
  wait_ring();  // K_1 and V_0 (and K_2, V_1 with the K look-ahead)
  ring_barrier();  // and every wave is done with slot 0 of K before K_R overwrites it
  if (FA_W_KPRE) {
#pragma unroll
    for (int i = 0; i < FA_W_PF; ++i) kpre[i] = k_frag(1, i);  // tile 0's block B: K_1
  }

  // ---- warming the L2 for the next workgroup --------------------------------------------
  // The hardware starts workgroup b + next_stride (the next round, same XCD, hence the
  // same L2) when a workgroup of this round ends, and every workgroup of a round would
  // fetch its 64 KB of Q from HBM at the same moment. So three tiles before its end this
  // workgroup copies that Q tile, and the first K tile of its head (the next workgroup
  // waits for both before its first MFMA), through the L2 into a scratch area of LDS;
  // the next workgroup then finds them in the cache. The copies join the ring's memory
  // counter: the waits of that iteration and the next leave them in flight as well.
  constexpr int WARM_Q = D / 8;   // 64 rows of Q per wave, 1 KB per copy
  constexpr int WARM_K = D / 32;  // 16 rows of K_0 per wave
  constexpr int WARM_OPS = WARM_Q + WARM_K;
  const int next_item = p.next_stride > 0 ? (int)blockIdx.x + p.next_stride : -1;
  const bool do_warm = next_item >= 0 && next_item < p.n_qt * p.BH && n_kt >= 4;
  const int j_warm = n_kt - 3;
  // buffer over `rows` rows of src from row r0 (rows past N read as zeros), wave-uniform:
  // read from the first lane so it stays in scalar registers
  auto rows_rsrc = [&](const uint16_t* src, int r0, int rows) {
    const u32x4_t r4 = buffer_rsrc((uint64_t)(uintptr_t)(src + (size_t)min(r0, N - 1) * D),
                                   (uint32_t)(max(min(N - r0, rows), 0) * D * 2));
    return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane(r4[0]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(r4[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(r4[2]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(r4[3])};
  };
  auto warm_next = [&]() {
    int bh2, qt2;
    decode_tile<CAUSAL>(p, next_item, bh2, qt2);
    const size_t head2 = (size_t)bh2 * (size_t)N * D;
    const u32x4_t rq = rows_rsrc(p.q + head2, qt2 * G::BR + wid * 64, 64);
    const u32x4_t rk = rows_rsrc(p.k + head2, wid * (BC / NW), BC / NW);
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(warm + wid * 64));
    const uint32_t off = (uint32_t)lane * 16u;  // 1 KB per copy: 64 lanes x 16 B
#pragma unroll
    for (int i = 0; i < WARM_Q; ++i) lds_copy16(rq, off + 1024u * i, lds, 0);
#pragma unroll
    for (int i = 0; i < WARM_K; ++i) lds_copy16(rk, off + 1024u * i, lds, 0);
  };
  static_assert(D * 2 * 64 == WARM_Q * 1024 && D * 2 * (BC / NW) == WARM_K * 1024,
                "one wave's rows are whole 1 KB copies");
  static_assert(NDMA * RING_LAG + WARM_OPS <= 63, "outstanding copies fit the vmcnt field");

  // ---- main loop: slots of tile j are j % R (K and V), unrolled over the ring --------
  for (int j0 = 0; j0 < n_kt; j0 += R) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int j = j0 + u;
      if (j >= n_kt) break;
      const Copies cp = {u, (u + R - 1) % R, j + R, j + R - 1};
      STile& s_cur = (u % 2 == 0) ? sa : sb;
      STile& s_nxt = (u % 2 == 0) ? sb : sa;
      if (do_warm && j == j_warm) warm_next();
      if (wave_live && j < w_kt)
        tile(s_cur, s_nxt, (u + 1) % R, u, (u + 2) % R, j, j + 1 < w_kt, cp);
      else
        copy_all(cp);
      if (do_warm && (j == j_warm || j == j_warm + 1))
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA * RING_LAG + WARM_OPS) : "memory");
      else
        wait_ring();
      ring_barrier();
    }
  }

  // The last iterations' copies (of clamped tiles that no iteration reads) may still be
  // in flight: let them land before the workgroup can end and its LDS be reassigned.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: O = O~ / l, L = (m*c + log2 l) * ln 2 ------------------------------
  // Under the causal mask the waves of a workgroup finish at different times: each
  // stores its rows directly (8-byte pieces) as soon as it is done. Without the mask they
  // finish together, and the rows go out through LDS as whole-row chunks (ai2048 +3%;
  // the barrier this needs cost 1.5% on long causal runs).
  if constexpr (CAUSAL) {
    if (!wave_live) return;
    const float kLn2 = 0.69314718055994530942f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      drain_o(qb);
      const float l_tot = xhalf_sum(ls[qb][0] + ls[qb][1]);
      const int qi = qbase[qb] + l32;
      if (qi < N) {
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
  } else {
    // O leaves through LDS: each wave writes its 64 rows (the accumulator layout gives a
    // lane 8 bytes of one row per write) into its own part of the K ring, then stores them
    // as 16-byte chunks of whole rows (a store instruction covers 64 / CPR whole rows),
    // instead of scattering 8-byte pieces over 32 rows per instruction. Chunk c of row r
    // sits at chunk c ^ (r % CPR) of the row, so neither side conflicts on banks. The
    // barrier makes every wave's last copies land before the ring is reused.
    static_assert(R * CHUNKS >= NW * 64 * CPR && (CPR & (CPR - 1)) == 0 && CPR <= 64,
                  "a 64-row O tile per wave fits the K ring");
    ring_barrier();
    if (!wave_live) return;
    const float kLn2 = 0.69314718055994530942f;
    unsigned char* ot = reinterpret_cast<unsigned char*>(kbuf + wid * 64 * CPR);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      drain_o(qb);
      const float l_tot = xhalf_sum(ls[qb][0] + ls[qb][1]);
      const float inv = 1.0f / l_tot;
      const int rr = 32 * qb + l32;  // row of the wave's tile
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& a = oacc[db][qb];
          const uint32_t w0 = E::pack(a[4 * g + 0] * inv, a[4 * g + 1] * inv);
          const uint32_t w1 = E::pack(a[4 * g + 2] * inv, a[4 * g + 3] * inv);
          const int c = db * 4 + g;  // 16-byte chunk of the row; this lane holds half hh
          *reinterpret_cast<u32x2_t*>(ot + (rr * CPR + (c ^ (rr & (CPR - 1)))) * 16 + hh * 8) =
              u32x2_t{w0, w1};
        }
      const int qi = qbase[qb] + l32;
      if (qi < N && hh == 0)
        p.lse[(size_t)bh * N + qi] = (ms[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own writes, in order
#pragma unroll
    for (int it = 0; it < CPR; ++it) {
      const int rr = (64 / CPR) * it + lane / CPR, c = lane % CPR;
      const u32x4_t x =
          *reinterpret_cast<const u32x4_t*>(ot + (rr * CPR + (c ^ (rr & (CPR - 1)))) * 16);
      const int qi = qbase[rr >> 5] + (rr & 31);
      if (qi < N) *reinterpret_cast<u32x4_t*>(p.o + head + (size_t)qi * D + c * 8) = x;
    }
  }
}

}  // namespace fa
