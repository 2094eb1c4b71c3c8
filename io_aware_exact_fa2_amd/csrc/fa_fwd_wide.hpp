// fa_fwd_wide.hpp — FA2-order attention forward for gfx950 (MI355X): one wave per
// SIMD, 64 queries per wave, head dims 64 and 128, with the key tiles in a three-stage
// pipeline and the rescale decided from row sums.
//
// Algorithm ([P1] currybab.bearblog.dev, "Triton으로 FlashAttention 구현하기 전에 -
// FA1, 2 forward pass", section "FlashAttention 2 forward pass 알고리즘 분석"): the
// query row block is the outer loop (one workgroup per query block, head and batch),
// key/value blocks stream through LDS in the inner loop, each row keeps its running
// max and sum on chip, rescales the unnormalised output by alpha = exp(m_old - m_new)
// only, and divides once at the end. Waves own disjoint query rows (split-Q). With
// SPLIT, workgroup (s, head, query block) covers only the keys of split s and writes its
// normalized partial O and partial L in float32 for the split-KV merge (fa_fwd_split.hpp).
//
// Why this kernel. With one wave per SIMD the wave issues everything itself, and the
// softmax's VALU work per tile (one FMA, one exponential, one add per score, half a
// pack) is almost as long as the tile's 64 MFMAs, so the wave is issue bound. The
// running max of each key tile (half a max3 per score, plus the cross-half exchange
// and the vote) is the one piece of that work the method does not need on every tile:
// the reference max only has to keep the probabilities bounded. Here a tile's softmax
// is computed against the current reference and its probabilities are summed per lane
// anyway; if every lane's tile sum is at most 2^tau, every probability is, and nothing
// else happens. Only when some lane's sum exceeds 2^tau (a probability may) does the
// wave take the row max of that tile, raise the references by the rule of the pages
// (alpha = exp(m_old - m_new) applied to l and O~, when the max exceeds the reference
// by more than tau) and recompute the tile's softmax. The softmax does not depend on
// the reference (the max shift cancels, [P1] "Online Softmax 개념"), so O and L are
// those of the per-block update up to rounding.
//
// The check must come before any P V product reads the tile's probabilities, so the
// tiles run in a three-stage pipeline: iteration j issues the S^T MFMAs of tile j+2,
// the P V MFMAs of tile j, and in between them the whole softmax of tile j+1, whose
// sums are checked at the end of the iteration; its P V products run in the next.
//
// gfx950 mapping: K and V tiles are copied HBM -> LDS by buffer_load_dwordx4 ... lds
// (no register staging) into a ring of R slots each; S^T = K Q^T and
// O^T = V^T P^T on v_mfma_f32_32x32x16_{bf16,f16}, each lane owning one query column,
// the S^T accumulator rounded to 16 bits is the B operand of P V (key rows enter with
// bits 2 and 3 of the row index swapped); XOR-swizzled LDS rows, transposed V reads
// (ds_read_b64_tr_b16), exp2 with log2(e) folded into the scale; fenced MFMA slots,
// each issuing one MFMA and then the work that runs while the matrix core executes it.
#pragma once

#include "fa_common.hpp"

#ifndef FA_W_PF
#define FA_W_PF 3  // MFMA steps an LDS operand read runs ahead
#endif

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
  static_assert(R >= 4 && R % 2 == 0, "the ring holds the tiles of three stages");
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The main loop's copies keep M0 one copy ahead: each issues its load with the LDS
// address the previous one left in M0, then sets M0 to the next copy's (saving the
// set-up and the wait state in front of every load). An LDS copy needs one instruction
// between the M0 write and itself; the loop's copies sit two MFMA slots apart, and
// callers that issue them back to back put an s_nop in between. Nothing else writes M0
// while the loop runs.
__device__ __forceinline__ void lds_copy16_chained(u32x4_t rsrc, uint32_t voff, uint32_t next_lds,
                                                   int next_off /* a constant after unrolling */) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds\n\ts_add_u32 m0, %2, %3"
               :: "v"(voff), "s"(rsrc), "s"(next_lds), "n"(next_off) : "m0", "scc");
}
__device__ __forceinline__ void set_m0(uint32_t lds, int off /* a constant */) {
  asm volatile("s_add_u32 m0, %0, %1" :: "s"(lds), "n"(off) : "m0", "scc");
}
#pragma clang diagnostic pop

// x = (c <= t) ? x : -inf, with c a constant after unrolling. Compare and select
// stay one pair, so no lane masks pile up in scalar registers across a tile.
__device__ __forceinline__ float keep_if_le(float x, int c, int t) {
  // v_cndmask reads VCC, so -inf comes from a register (one constant-bus operand)
  asm("v_cmp_le_i32 vcc, %2, %1\n\tv_cndmask_b32 %0, %3, %0, vcc"
      : "+v"(x) : "v"(t), "n"(c), "v"(-__builtin_inff()) : "vcc");
  return x;
}


// The softmax of one key tile, as a stream of VALU instructions ("ops") placed into the
// MFMA slots of an iteration. A lane holds NPAIR pairs of scores per tile; per pair, ops
// 0-1 are the two exponent arguments s c - m (FMA), 2-3 their exponentials, 4-5 the two
// adds into the tile sums, 6 the 16-bit pack into the P operand. A query block's tile
// sums start as the sums of its first two pairs (op 4 adds the pair, op 5 is dropped), so
// no pair's probability is merely copied into a sum. The three stages of
// consecutive pairs are staggered (step k holds the arguments of pair k, the
// exponentials of pair k - LB and the sums and pack of pair k - LC), so an op never
// reads the result of the op just before it. The ops go into the slots in stream order
// such that the issue time of every slot (its ops plus its LDS reads and copies, in
// half-cycles of measured issue cost) is as even as possible.
template <int NPAIR, int NSLOT>
struct OpSched {
  int code[7 * NPAIR];  // 8 * pair + op
  int n;                // ops in the stream
  int first[NSLOT + 1]; // ops [first[s], first[s + 1]) go into slot s
};
// Pairs 0, 1 (query block 0) and 4, 5 (query block 1) start the two tile sums of their
// query block: pair v's scores sit in registers 8 (v / 8) + 2 (v % 4) of query block
// (v / 4) % 2.
constexpr bool sum_starter(int v) { return v < 8 && v % 4 < 2; }
template <int NPAIR, int NSLOT, int LB, int LC, int SC_N, int NQK, int NPV, int PF, int NDMA>
constexpr OpSched<NPAIR, NSLOT> make_op_sched() {
  OpSched<NPAIR, NSLOT> t{};
  int n = 0;
  const int lag[3] = {0, LB, LC};
  const int ops_of[3][4] = {{0, 1, -1, -1}, {2, 3, -1, -1}, {4, 5, 6, -1}};
  for (int k = 0; k < NPAIR + LC; ++k)
    for (int st = 0; st < 3; ++st) {
      const int v = k - lag[st];
      if (v < 0 || v >= NPAIR) continue;
      for (int q = 0; q < 4 && ops_of[st][q] >= 0; ++q)
        if (!(ops_of[st][q] == 5 && sum_starter(v))) t.code[n++] = 8 * v + ops_of[st][q];
    }
  t.n = n;
  // issue costs in half-cycles
  const int op_cost[7] = {11, 11, 24, 24, 11, 11, 11};
  int fixed[NSLOT] = {};
  long total = 0;
  for (int sl = 0; sl < NSLOT; ++sl) {
    int f = 4;  // the MFMA
    if (sl < SC_N) {
      const int i = sl / 2, qb = sl % 2;
      if (i + PF < NPV) f += 8;                       // one transposed V read
      if (qb == 0 && i >= NPV - PF) f += 8;           // a K read for the next block
      if (sl % 2 == 1 && sl / 2 < NDMA) f += 18;      // an LDS copy and its M0 set-up
    } else {
      const int sb = sl - SC_N, i = sb / 2, qb = sb % 2;
      if (qb == 0 && i + PF < NQK) f += 8;            // a K read
      if (i >= NQK - PF) f += 8;                      // a V^T read for the next iteration
    }
    fixed[sl] = f;
    total += f;
  }
  for (int i = 0; i < n; ++i) total += op_cost[t.code[i] % 8];
  long cum = 0;
  int o = 0;
  for (int sl = 0; sl < NSLOT; ++sl) {
    t.first[sl] = o;
    cum += fixed[sl];
    const long target = total * (sl + 1) / NSLOT;
    // take ops while that brings the running issue time closer to the target
    while (o < n) {
      const int c = op_cost[t.code[o] % 8];
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
template <int NPAIR, int NSLOT, int LB, int LC, int SC_N, int NQK, int NPV, int PF, int NDMA>
constexpr OpSched<NPAIR, NSLOT> kOpSched =
    make_op_sched<NPAIR, NSLOT, LB, LC, SC_N, NQK, NPV, PF, NDMA>();

template <bool BF16, int D, bool CAUSAL, int BC, int R, bool SPLIT = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fa_fwd_wide_kernel(const Params p) {
  using G = WideGeom<D, BC, R>;
  using E = Elt<BF16>;
  constexpr int NW = G::NW, CPR = G::CPR, NQK = G::NQK, NPV = G::NPV, NST = G::NST;
  constexpr int CHUNKS = G::CHUNKS, PW = G::PER_WAVE, NDMA = 2 * PW;
  constexpr int SB_N = 2 * NQK;                 // slots of the S^T block (tile j+2)
  constexpr int SC_N = 2 * NPV;                 // slots of the P V block (tile j)
  constexpr int NSLOT = SB_N + SC_N;
  constexpr int NPAIR = BC / 2;                 // score pairs per lane and tile
  constexpr int PF = FA_W_PF;                   // MFMA steps an LDS operand read runs ahead
  static_assert(R >= 4 && R % 2 == 0, "the ring holds the tiles of three stages");
  __shared__ __attribute__((aligned(1024))) u32x4_t kbuf[R * CHUNKS];
  __shared__ __attribute__((aligned(1024))) u32x4_t vbuf[R * CHUNKS];

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

  const int q0 = qt * G::BR;
  // wave w owns the 32-query blocks w and 7 - w of the workgroup's 256 queries
  const int qbase[2] = {q0 + 32 * wid, q0 + 32 * (2 * NW - 1 - wid)};
  const int wq0 = qbase[0];
  const int q_end = min(q0 + G::BR, N);
  const int n_kt = CAUSAL ? (min(q_end - kofs, Nk) + BC - 1) / BC : (Nk + BC - 1) / BC;
  // Splits start at multiples of the query tile, so under the causal mask a split either
  // starts at or before q0 (every query of the tile sees its first key) or after the
  // tile's last query: empty (n_kt <= 0), partial L = -inf and partial O = 0. An empty
  // split's workgroup runs the prologue on empty buffers (its copies read no memory), no
  // iteration, and writes those values; an early return here, or a loop known to run
  // at least once, would cost the loop registers.
  const bool empty = SPLIT && n_kt <= 0;
  const bool wave_live = wq0 < N;
  const int w_last_q = min(qbase[1] + 32, N) - 1;
  const int w_kt = empty ? 0 : CAUSAL ? min(n_kt, (w_last_q - kofs) / BC + 1) : n_kt;
  // the first tile that reaches past the keys or, under the causal mask, past the wave's
  // first query (key t BC + BC - 1 > wq0), and the number of the wave's tiles from there on
  const int t_mask = CAUSAL ? min(Nk / BC, (wq0 - kofs + 1) / BC) : Nk / BC;
  const uint32_t n_masked = (uint32_t)max(w_kt - t_mask, 0);

  // ---- HBM -> LDS copies: lane l of a wave's copy i of a tile writes 16-byte chunk
  // position (NW i + wid) * 64 + l of the tile (row-major, CPR chunks per row) and
  // fetches the row's logical chunk that the swizzle puts there ---------------------
  constexpr uint32_t II_BYTES = NW * 64 * 16;
  static_assert((NW * 64 / CPR) % 16 == 0, "copies are whole 16-row groups");
  uint32_t koff, voff;
  {
    const int f = wid * 64 + lane, row = f / CPR, ph = f % CPR;
    koff = (uint32_t)(row * D + (ph ^ swz_k<D>(row)) * 8) * 2u;
    voff = (uint32_t)(row * D + (ph ^ swz_v<D>(row)) * 8) * 2u;
  }
  // the buffer of tile t spans its rows below N (the range check zero-fills the rest);
  // a tile past the last (the pipeline's drain reads it and drops the results) has an
  // empty buffer, so its copies write zeros and read no memory
  auto tile_rsrc = [&](const uint16_t* src, int t) {
    const int k0 = min(t, n_kt - 1) * BC;
    return buffer_rsrc((uint64_t)(uintptr_t)(src + (size_t)k0 * D),
                       t < n_kt ? (uint32_t)(min(Nk - k0, BC) * D * 2) : 0u);
  };
  const uint32_t k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(kbuf + wid * 64));
  const uint32_t v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(vbuf + wid * 64));
  // copy step i of tile kt (K, into ring slot ks) and tile vt (V, slot vs): K copies
  // first, then V copies; the slots are compile-time constants after unrolling
  auto copy_step = [&](int kt, int ks, int vt, int vs, int i) __attribute__((always_inline)) {
    if (i < PW)
      lds_copy16(tile_rsrc(kg, kt), koff + II_BYTES * i, k_lds, ks * CHUNKS * 16 + i * NW * 1024);
    else if (i < NDMA)
      lds_copy16(tile_rsrc(vg, vt), voff + II_BYTES * (i - PW), v_lds,
                 vs * CHUNKS * 16 + (i - PW) * NW * 1024);
  };
  auto copy_k = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PW; ++i) copy_step(kt, kt % R, 0, 0, i);
  };
  auto copy_v = [&](int vt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = PW; i < NDMA; ++i) copy_step(0, 0, vt, vt % R, i);
  };
  // The loop's copies: iteration u of the group of R iterations that starts at tile j0
  // copies K_{j0+u+R+1} into ring slot (u+1) % R and V_{j0+u+R-1} into slot (u+R-1) % R.
  // Their buffers are taken relative to the group's base (tile j0's address kgj / vgj,
  // and remj, the bytes of rows below the last tile's end from tile j0 on): a tile's
  // buffer then reaches from its first row to that end, so rows past N, and tiles past
  // the last, read as zeros as above. (The address's high word is used as it is: device
  // addresses stay below 2^48, so it never reaches the resource's stride field.)
  constexpr uint32_t TB = (uint32_t)CHUNKS * 16u;  // bytes of a K (or V) tile
  // (an empty split has n_kt <= 0: no bytes)
  const int kv_rows = SPLIT ? max(min(n_kt * BC, Nk), 0) : min(n_kt * BC, Nk);
  const uint32_t kv_bytes = (uint32_t)kv_rows * (uint32_t)(D * 2);
  const uint16_t* kgj = kg;
  const uint16_t* vgj = vg;
  uint32_t remj = kv_bytes;
  auto rsrc_rel = [&](const uint16_t* base, int dt) __attribute__((always_inline)) {
    const uint64_t a = (uint64_t)(uintptr_t)base + (uint64_t)dt * TB;
    // max(remj, o) - o on the scalar unit (the compiler would saturate on the VALU)
    uint32_t size;
    asm("s_max_u32 %0, %1, %2\n\ts_sub_u32 %0, %0, %2"
        : "=&s"(size) : "s"(remj), "n"(dt * TB) : "scc");
    return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32), size, (uint32_t)kBufferWord3};
  };
  // copy i of iteration u (K copies first); M0 holds its LDS address and is then set to
  // the next copy's: copy i + 1, or copy 0 of iteration u + 1
  auto copy_loop = [&](int u, int i) __attribute__((always_inline)) {
    const int ks = (u + 1) % R, vs = (u + R - 1) % R;
    if (i < PW) {
      const u32x4_t rs = rsrc_rel(kgj, u + R + 1);
      if (i + 1 < PW)
        lds_copy16_chained(rs, koff + II_BYTES * i, k_lds, ks * CHUNKS * 16 + (i + 1) * NW * 1024);
      else
        lds_copy16_chained(rs, koff + II_BYTES * i, v_lds, vs * CHUNKS * 16);
    } else if (i < NDMA) {
      const u32x4_t rs = rsrc_rel(vgj, u + R - 1);
      const int iv = i - PW;
      if (i + 1 < NDMA)
        lds_copy16_chained(rs, voff + II_BYTES * iv, v_lds,
                           vs * CHUNKS * 16 + (iv + 1) * NW * 1024);
      else
        lds_copy16_chained(rs, voff + II_BYTES * iv, k_lds, ((u + 2) % R) * CHUNKS * 16);
    }
  };

  // ---- Q fragments (B operands of S^T = K Q^T), in AGPRs for the whole loop ----------
  // The wave's 64 Q rows (query block 0, then 1; rows past N repeat row N - 1, never
  // stored) go HBM -> LDS like the K tiles, in whole 1 KB copies, into the wave's slot of
  // the V ring (idle until V_0 is copied, after the prologue's first barrier): copy i,
  // lane l moves chunk position (64 i + l) % CPR of wave row (64 i + l) / CPR, which
  // holds the row's logical chunk position ^ swz_k(row), as in a K tile. Then the wave
  // reads its fragments from there, conflict-free as the K operand reads.
  // Prologue copies after the Q rows: K_0 .. K_3; V_0 .. V_2 follow the first barrier,
  // K_4 the second one (once every wave is done with K_0's slot).
  u32x4_t qf[2][D / 16];
  const uint32_t q_lds =  // slot wid of the V ring
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(vbuf + wid * CHUNKS));
  {
    static_assert(64 * CPR == CHUNKS, "a wave's Q rows fill one ring slot");
    const u32x4_t rq = buffer_rsrc((uint64_t)(uintptr_t)qg, (uint32_t)N * D * 2);
    // (an opaque copy of the lane index keeps these row numbers from being shared with
    // the epilogue's, which would hold them in registers across the whole loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int f = 64 * i + ln, r = f / CPR, ph = f % CPR;
      const int qi = min(qbase[r / 32] + (r % 32), N - 1);
      lds_copy16(rq, (uint32_t)(qi * D + (ph ^ swz_k<D>(r)) * 8) * 2u, q_lds, i * 1024);
    }
  }
  copy_k(0);
  copy_k(1);
  copy_k(2);
  copy_k(3);

  // ---- running state ---------------------------------------------------------------
  f32x16_t oacc[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][qb][r] = 0.f;
  float ms[2] = {0.f, 0.f};                   // reference max per query block (log2 units)
  float ls[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // running sums, two chains per query block
  float ts[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // sums of the tile in the softmax stage
  const float c = p.c;
  const float thr = __builtin_amdgcn_exp2f(p.tau);  // largest probability allowed

  // ---- per-lane LDS read addresses: lane l reads K tile row key_of_row(l % 32), chunk
  // 2 ds + l / 32 (the ds step folds in by XOR), and V^T transposed, 4 rows x 4 chunks
  // per 16-lane group ---------------------------------------------------------------
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
  auto k_frag = [&](int slot, int i) __attribute__((always_inline)) {
    const int kb = i % (BC / 32), ds = i / (BC / 32);
    return *(lds_u32x4_t*)(uintptr_t)((kaddr0 ^ (uint32_t)(ds << 5)) + slot * CHUNKS * 16 +
                                      kb * 32 * CPR * 16);
  };
  auto v_half = [&](int slot, int i, int h) __attribute__((always_inline)) {
    const int db = i % (D / 32), st = i / (D / 32);
    const uint32_t b = vaddr[db] + slot * CHUNKS * 16;
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (lds_s16x4_t*)(uintptr_t)(b + (16 * st + 4 * h) * CPR * 16)));
  };

  typedef f32x16_t STile[BC / 32][2];
  typedef u32x4_t PTile[2][NST];  // P~ packed as P V operands: [query block][16-key step]
  auto zero = [](STile& s) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
  };
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

  // S^T of tile t with its K rows read from global memory (the tile's ring slot may
  // already hold a later tile): same operands, same accumulation order as qk_plain, so
  // the same bits. Rows past the last key read the last key; the mask clears them.
  auto qk_global = [&](int t, STile& s) {
    zero(s);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int kb = i % (BC / 32), ds = i / (BC / 32);
      const int row = min(t * BC + kb * 32 + key_of_row(l32), Nk - 1);
      const u32x4_t kf = ld16(kg + (size_t)row * D + ds * 16 + hh * 8);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = E::mfma(kf, qf[qb][ds], s[kb][qb]);
    }
  };

  // -inf on keys past the last one and, under the causal mask, on keys after the query;
  // only tiles that reach past the keys or cross the diagonal need it
  auto mask = [&](STile& s, int j) __attribute__((always_inline)) {
    // tiles [t_mask, w_kt) need it (tiles past the wave's last one are never used)
    if ((uint32_t)(j - t_mask) >= n_masked) return;
    const int base = j * BC + 8 * hh;
    // wait out the S^T MFMAs before the inline-assembly compares read their results
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0][0]));
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        if (kb + qb > 0) asm volatile("" : "+v"(s[kb][qb]));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int last = CAUSAL ? min(Nk - 1, qbase[qb] + l32 - kofs) : Nk - 1;
      const int t = last - base;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][qb][r] = keep_if_le(s[kb][qb][r], kb * 32 + key_of_reg(r, 0), t);
    }
  };

  // ---- softmax of one tile: the op stream of make_op_sched -----------------------------
  // A pair's exponent arguments and exponentials wait in tq / pq (indexed by the pair,
  // modulo the pairs in flight between the stages); the first pair of each query block
  // assigns the tile sums, the others add to them. Results are pinned, so each op is
  // computed in the slot that issues it.
  constexpr int LB = 1, LC = 2, NTQ = LB + 1, NPQ = LC - LB + 1;
  float tq[NTQ][2], pq[NPQ][2];
#define FA_W_OPS kOpSched<NPAIR, NSLOT, LB, LC, SC_N, NQK, NPV, PF, NDMA>
  // op o of the stream: see make_op_sched
  auto exp_op = [&](const STile& s, PTile& pt, int o) __attribute__((always_inline)) {
    const int v = FA_W_OPS.code[o] / 8, op = FA_W_OPS.code[o] % 8;
    const int qb = (v / 4) % 2, e = 8 * (v / 8) + 2 * (v % 4);
    const int bt = v % NTQ, bp = v % NPQ;
    if (op < 2) {
      tq[bt][op] = __builtin_fmaf(s[(e + op) / 16][qb][(e + op) % 16], c, -ms[qb]);
      asm volatile("" : "+v"(tq[bt][op]));
    } else if (op < 4) {
      // c > 0 on this path, so a masked score (-inf) gives exp2(-inf) = 0 exactly
      pq[bp][op - 2] = __builtin_amdgcn_exp2f(tq[bt][op - 2]);
      asm volatile("" : "+v"(pq[bp][op - 2]));
    } else if (op < 6) {
      if (sum_starter(v))  // op 4 only: sum v % 2 of the query block starts as the pair's
        ts[qb][v % 2] = pq[bp][0] + pq[bp][1];
      else
        ts[qb][op - 4] += pq[bp][op - 4];
      asm volatile("" : "+v"(ts[qb][sum_starter(v) ? v % 2 : op - 4]));
    } else {
      uint32_t w = E::pack(pq[bp][0], pq[bp][1]);
      asm volatile("" : "+v"(w));
      pt[qb][e / 8][(e % 8) / 2] = w;
    }
  };
  auto softmax_all = [&](const STile& s, PTile& pt) __attribute__((always_inline)) {
#pragma unroll
    for (int o = 0; o < FA_W_OPS.n; ++o) exp_op(s, pt, o);
  };

  // O~ in AGPRs is written by inline-assembly MFMAs the compiler does not track: pad
  // before any VALU access (an 8-pass XDL result needs about a dozen wait states)
  auto drain_o = [&](int qb) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(oacc[0][qb]));
#pragma unroll
    for (int db = 1; db < D / 32; ++db) asm volatile("" : "+a"(oacc[db][qb]));
  };
  // m_new = max(m_old, rowmax) when some row of the wave's query block exceeds its
  // reference by more than tau (need); alpha = exp2(m_old - m_new) rescales l and O~
  auto grow_max = [&](int qb, float mxs, uint64_t need) {
    if (need != 0) {
      const float ms_new = __builtin_fmaxf(ms[qb], mxs);
      const float alpha = __builtin_amdgcn_exp2f(ms[qb] - ms_new);
      ms[qb] = ms_new;
      ls[qb][0] *= alpha;
      ls[qb][1] *= alpha;
      drain_o(qb);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
        asm volatile("" : "+a"(oacc[db][qb]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto row_max = [&](const STile& s, int qb) {
    float m0 = -__builtin_inff(), m1 = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        m0 = __builtin_fmaxf(m0, __builtin_fmaxf(s[kb][qb][r], s[kb][qb][r + 1]));
        m1 = __builtin_fmaxf(m1, __builtin_fmaxf(s[kb][qb][r + 2], s[kb][qb][r + 3]));
      }
    return xhalf_max(__builtin_fmaxf(m0, m1)) * c;
  };
  // Tile t in the softmax stage may hold a probability above 2^tau (some lane's tile
  // sum exceeds it): recompute its scores (the softmax stage has consumed the S^T tile
  // by now, so it need not stay in registers for this rare case), take their row max,
  // raise the references that the rule raises, and recompute the tile's softmax.
  auto fix_tile = [&](int t, PTile& pt) {
    STile sx;
    qk_global(t, sx);
    mask(sx, t);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mx = row_max(sx, qb);
      grow_max(qb, mx, __builtin_amdgcn_ballot_w64(mx > ms[qb] + p.tau));
    }
    softmax_all(sx, pt);
  };
  // Tile sums checked: all at most 2^tau, or tile t is fixed. Then they join l.
  auto settle = [&](int t, PTile& pt) __attribute__((always_inline)) {
    const float big = __builtin_fmaxf(__builtin_fmaxf(ts[0][0], ts[0][1]),
                                      __builtin_fmaxf(ts[1][0], ts[1][1]));
    if (__builtin_amdgcn_ballot_w64(!(big <= thr)) != 0) fix_tile(t, pt);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      ls[qb][0] += ts[qb][0];
      ls[qb][1] += ts[qb][1];
    }
  };

  // ---- one iteration: P V of tile j, softmax of tile j+1, S^T of tile j+2 -------------
  // Slots 0 .. SC_N-1 issue the P V MFMAs (step i = slot / 2: head-dim block i % (D/32),
  // 16-key step i / (D/32); query block slot % 2), slots SC_N .. NSLOT-1 the S^T MFMAs
  // (step i: key block i % (BC/32), head-dim slice i / (BC/32)). P V first: the P tile
  // it consumes dies while the next one is produced, and the S^T tile it produces is
  // born after half the softmax tile has been consumed, which keeps the live registers
  // down. The softmax ops of tile j+1 are spread over all slots. LDS operand
  // reads run PF steps ahead: the first K operands of the S^T block are read in the
  // last P V slots, the first V^T operands of the next iteration in the last S^T slots
  // (from a slot no copy of the next iteration touches). This wave's copies of K_{j+R+1}
  // and V_{j+R-1} (into the slots of K_{j+1} and V_{j-1}, both read in the previous
  // iteration) go into every second slot of the P V block, early in the iteration: a V
  // tile is first read at the end of the iteration after next, so it has nearly two
  // iterations to land.
  // On a wave's last tile the softmax stage works on a stale tile and its results are
  // dropped (no branch inside the slots).
  constexpr int COPY_EVERY = 2;
  static_assert(COPY_EVERY * NDMA <= SC_N, "copies spread over the P V block");
  u32x4_t vq[PF];  // the first V^T operands of the next P V block
  auto iteration = [&](int u, int j, STile& s_new, const STile& s_mid, PTile& p_mid,
                       const PTile& p_cur) __attribute__((always_inline)) {
    // ring slots: tile t is in slot t % R, and j % R = u
    const int vst = u, kst = (u + 2) % R, vnext = (u + 1) % R;
    u32x4_t vf[NPV];
    u32x4_t kf[NQK];
#pragma unroll
    for (int i = 0; i < PF; ++i) vf[i] = vq[i];
#pragma unroll
    for (int sc = 0; sc < SC_N; ++sc) {
      const int i = sc / 2, qb = sc % 2, db = i % (D / 32), st = i / (D / 32);
      // keep the previous step's sources live until this step (the inline-assembly
      // MFMAs read them over several cycles)
      if (qb == 0 && i > 0)
        asm volatile("" ::"v"(vf[i - 1]), "v"(p_cur[0][(i - 1) / (D / 32)]),
                     "v"(p_cur[1][(i - 1) / (D / 32)]));
      // one LDS wait per two steps: the operands of steps i and i + 1 together (read
      // PF and PF - 1 steps before)
      if (qb == 0 && i % 2 == 0 && i + 1 < NPV) asm volatile("" ::"v"(vf[i]), "v"(vf[i + 1]));
      mfma_acc_agpr<BF16>(oacc[db][qb], vf[i], p_cur[qb][st]);
      __builtin_amdgcn_sched_barrier(0);
      if (i + PF < NPV) {
        const u32x2_t h = v_half(vst, i + PF, qb);
        vf[i + PF][2 * qb] = h[0];
        vf[i + PF][2 * qb + 1] = h[1];
      }
      if (qb == 0 && i >= NPV - PF) kf[i - (NPV - PF)] = k_frag(kst, i - (NPV - PF));
      if (sc % COPY_EVERY == 1) copy_loop(u, sc / COPY_EVERY);
#pragma unroll
      for (int o = FA_W_OPS.first[sc]; o < FA_W_OPS.first[sc + 1]; ++o) exp_op(s_mid, p_mid, o);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"v"(vf[NPV - 1]), "v"(p_cur[0][NST - 1]), "v"(p_cur[1][NST - 1]));
    zero(s_new);
#pragma unroll
    for (int sb = 0; sb < SB_N; ++sb) {
      const int sl = SC_N + sb;
      const int i = sb / 2, qb = sb % 2, kb = i % (BC / 32), ds = i / (BC / 32);
      if (qb == 0 && i % 2 == 0 && i + 1 < NQK) {
        asm volatile("" ::"v"(kf[i]), "v"(kf[i + 1]));
        __builtin_amdgcn_sched_barrier(0);  // (the product must not move above the wait)
      }
      s_new[kb][qb] = E::mfma(kf[i], qf[qb][ds], s_new[kb][qb]);
      __builtin_amdgcn_sched_barrier(0);
      if (qb == 0 && i + PF < NQK) kf[i + PF] = k_frag(kst, i + PF);
      if (i >= NQK - PF) {
        const u32x2_t h = v_half(vnext, i - (NQK - PF), qb);
        vq[i - (NQK - PF)][2 * qb] = h[0];
        vq[i - (NQK - PF)][2 * qb + 1] = h[1];
      }
#pragma unroll
      for (int o = FA_W_OPS.first[sl]; o < FA_W_OPS.first[sl + 1]; ++o) exp_op(s_mid, p_mid, o);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask(s_new, j + 2);
  };

  // ---- ring waits and barriers --------------------------------------------------------
  // At the end of iteration j every copy but this iteration's must have landed (the next
  // iteration reads K_{j+3}, V_{j+1}, and at its end V_{j+2}), and the barrier must follow
  // this wave's last K read (the 2 PF V^T reads for the next iteration issued
  // after it may stay in flight: no copy of the next iteration goes into their slot).
  auto end_wait = [&]() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory"); };
  auto ring_barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  auto loop_barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(2 * PF) : "memory");
  };

  // ---- prologue: S^T and softmax of tile 0, S^T of tile 1 -----------------------------
  STile sa, sb;
  PTile pa, pb;
  // Q, K_0 and K_1 have landed (K_2 and K_3 may be in flight)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PW) : "memory");
  {
    // wave row 32 qb + l32, logical chunk 2 ds + hh (16 columns ds, half hh)
    const uint32_t qaddr = (uint32_t)(uintptr_t)vbuf + (uint32_t)(wid * CHUNKS * 16) +
                           (uint32_t)((l32 * CPR + (hh ^ swz_k<D>(l32))) * 16);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        qf[qb][ds] = *(lds_u32x4_t*)(uintptr_t)((qaddr ^ (uint32_t)(ds << 5)) + qb * 32 * CPR * 16);
        qf[qb][ds] ^= p.qsign;
        asm volatile("" : "+a"(qf[qb][ds]));
      }
  }
  ring_barrier();  // every wave has its Q fragments: the V ring is free for V_0 .. V_2
  copy_v(0);
  copy_v(1);
  copy_v(2);
  if (wave_live) {
    qk_plain(0, sa);
    mask(sa, 0);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) ms[qb] = row_max(sa, qb);  // tile 0 holds key 0: finite
    // S^T of tile 1 with the softmax of tile 0 in its slots
    zero(sb);
    u32x4_t kf[NQK];
#pragma unroll
    for (int i = 0; i < PF; ++i) kf[i] = k_frag(1, i);
#pragma unroll
    for (int sl = 0; sl < SB_N; ++sl) {
      const int i = sl / 2, qb = sl % 2, kb = i % (BC / 32), ds = i / (BC / 32);
      sb[kb][qb] = E::mfma(kf[i], qf[qb][ds], sb[kb][qb]);
      __builtin_amdgcn_sched_barrier(0);
      if (qb == 0 && i + PF < NQK) kf[i + PF] = k_frag(1, i + PF);
#pragma unroll
      for (int o = FA_W_OPS.n * sl / SB_N; o < FA_W_OPS.n * (sl + 1) / SB_N; ++o)
        exp_op(sa, pa, o);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask(sb, 1);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      ls[qb][0] = ts[qb][0];
      ls[qb][1] = ts[qb][1];
    }
  }
  // every wave is done with K_0's slot before K_R goes into it
  ring_barrier();
  copy_k(R);
  set_m0(k_lds, (1 % R) * CHUNKS * 16);  // the loop's first copy: K_{R+1}, ring slot 1
  // everything but K_R has landed: K_2 .. K_{R-1}, V_0 .. V_2
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PW) : "memory");
  ring_barrier();
#pragma unroll
  for (int i = 0; i < PF; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x2_t x = v_half(0, i, h);
      vq[i][2 * h] = x[0];
      vq[i][2 * h + 1] = x[1];
    }

  // ---- main loop: iteration j = tile j's P V; unrolled over the ring -------------------
  // S^T tiles alternate between sa and sb (tile t in sa when t is even), P tiles
  // between pa and pb likewise; with R even, the parity of j is that of u.
  for (int j0 = 0; j0 < n_kt; j0 += R) {
    kgj = kg + (size_t)j0 * BC * D;
    vgj = vg + (size_t)j0 * BC * D;
    remj = kv_bytes - (uint32_t)j0 * TB;  // j0 < n_kt: tile j0 starts below the end
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int j = j0 + u;
      if (j >= n_kt) break;
      STile& s_mid = (u % 2 == 0) ? sb : sa;  // tile j+1
      STile& s_new = (u % 2 == 0) ? sa : sb;  // tile j+2
      PTile& p_cur = (u % 2 == 0) ? pa : pb;  // tile j
      PTile& p_mid = (u % 2 == 0) ? pb : pa;  // tile j+1
      if (wave_live && j < w_kt) {
        iteration(u, j, s_new, s_mid, p_mid, p_cur);
        if (j + 1 < w_kt) settle(j + 1, p_mid);
      } else {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
          asm volatile("s_nop 0");  // the wait state after the previous copy's M0 write
          copy_loop(u, i);
        }
      }
      end_wait();
      loop_barrier();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: O = O~ / l, L = (m*c + log2 l) * ln 2 ------------------------------
  if constexpr (SPLIT) {
    // the split's normalized partial O (float32) and partial L, straight from registers:
    // lane (query qbase[qb] + l32, half hh) holds head dims 32 db + 8 g + 4 hh + 0..3
    if (!wave_live) return;
    const float kLn2 = 0.69314718055994530942f;
    // (an opaque copy of the lane index keeps the row addresses below from being computed
    // before the loop and held in registers across it)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      drain_o(qb);
      const float l_tot = xhalf_sum(ls[qb][0] + ls[qb][1]);
      const float inv = empty ? 0.f : 1.0f / l_tot;  // an empty split's O~ is 0
      const int qi = qbase[qb] + (ln & 31);
      if (qi < N) {
        const size_t row = ((size_t)split * p.BH + bh) * N + qi;
        float* prow = p.o_part + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = oacc[db][qb];
            *reinterpret_cast<float4*>(prow + db * 32 + g * 8 + (ln >> 5) * 4) =
                float4{a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv};
          }
        if (ln < 32)
          p.l_part[row] = empty ? -__builtin_inff() : (ms[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
      }
    }
    return;
  } else {
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
      const int rr = 32 * qb + l32;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16_t& a = oacc[db][qb];
          const uint32_t w0 = E::pack(a[4 * g + 0] * inv, a[4 * g + 1] * inv);
          const uint32_t w1 = E::pack(a[4 * g + 2] * inv, a[4 * g + 3] * inv);
          const int cc = db * 4 + g;
          *reinterpret_cast<u32x2_t*>(ot + o_half_off<CPR>(rr, cc, hh)) = u32x2_t{w0, w1};
        }
      const int qi = qbase[qb] + l32;
      if (qi < N && hh == 0)
        p.lse[(size_t)bh * N + qi] = (ms[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int it = 0; it < CPR; ++it) {
      const int rr = (64 / CPR) * it + lane / CPR, cc = lane % CPR;
      const u32x4_t x = o_chunk_read<CPR>(ot, rr, cc);
      const int qi = qbase[rr >> 5] + (rr & 31);
      if (qi < N) *reinterpret_cast<u32x4_t*>(p.o + head + (size_t)qi * D + cc * 8) = x;
    }
  }
}

#undef FA_W_OPS
}  // namespace fa
