// fa_bwd.hpp — backward pass of the attention forward in fa_fwd_*.hpp, for gfx950.
//
// What the pages fix ([P1] currybab.bearblog.dev, FA2 section, the LSE identity; [P2]
// iq-universe.github.io, "FlashAttention: SRAM tiling으로 O(N²) HBM을 우회하다", the
// activation-memory paragraph; [P3] ariser.io, "계산을 다시 하는 편이 싸다는 역설"): the
// forward keeps only O and the per-row logsumexp L, and the backward recomputes the
// probabilities block by block, P_ij = exp(S_ij - L_i), instead of storing the N x N
// matrix. The gradients are the chain rule of the forward definition (for the loss
// sum(O * dO)):
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = rowsum(dO * O)_i,
//     dQ = scale dS K,  dK = scale dS^T Q.
// Three kernels in stream order, so that every output is written by exactly one
// workgroup (no atomics and no workspace beyond the outputs):
//   * fa_bwd_delta_kernel: D once per row from dO and O, into the dQ output's memory
//     (before dQ is written there);
//   * fa_bwd_dkdv_kernel: one workgroup per 128 keys (32 per wave) walks the query
//     tiles, recomputing S and dP with the key on the lane, and accumulates
//     dV^T = dO^T P and dK^T = Q^T dS, reading D;
//   * fa_bwd_dq_kernel: one workgroup per 128 query rows (32 per wave) walks the key
//     tiles, recomputing S^T and dP^T with the row on the lane (as in the forward), and
//     accumulates dQ^T = K^T dS^T; it computes D for its own rows and then overwrites
//     that memory with dQ.
// All products run on
// v_mfma_f32_32x32x16_{bf16,f16}; an accumulator becomes a 16-bit B operand of the next
// product by the row permutation of the forward kernels (bits 2 and 3 of the MFMA row
// swapped). Tiles are staged in LDS by buffer-to-LDS copies into two buffers, the next
// tile's copies in flight while the current one is computed, with a swizzle that keeps
// both the row reads and the transposed reads (ds_read_b64_tr_b16) free of bank
// conflicts.
#pragma once

#include "fa_common.hpp"

// d = 128 dK/dV: issue both 32-query blocks' S and dP products before either block's
// softmax terms (1, measured +2-4%) or one block at a time (0)
#ifndef FA_BWD_PIPE
#define FA_BWD_PIPE 1
#endif
// dQ: an interleave pattern for the machine scheduler that keeps the LDS operand reads
// FA_BWD_DQ_AHEAD products ahead of the MFMAs that use them (1, measured +1-2%)
#ifndef FA_BWD_DQ_SG
#define FA_BWD_DQ_SG 1
#endif
#ifndef FA_BWD_DQ_AHEAD
#define FA_BWD_DQ_AHEAD 2
#endif
// dK/dV and dQ: the slot-scheduled kernels of fa_bwd_wide.hpp (1) or the kernels here (0)
#ifndef FA_BWD_WIDE
#define FA_BWD_WIDE 1
#endif

namespace fa {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;  // [BH, N] D_i = rowsum(dO * O); lives in dq's memory until dQ is written
  float* lse2;   // [BH, N] L_i log2(e), next to delta in dq's memory
  int N;
  int BH;
  float scale;  // signed
  float c;      // scale * log2(e), signed
};

// XOR swizzle of the 16-byte chunks of LDS row `row` of a staged tile. The tiles are
// read two ways: as MFMA row operands (16 lanes read one logical chunk of 16
// consecutive rows) and transposed with ds_read_b64_tr_b16 (a half-wave reads 4
// consecutive rows x 4 consecutive chunks). Both are bank-conflict free when the
// swizzle is a bijection of the rows within a 256-byte bank line (d = 128: rows
// 0..15; d = 64: the 8 rows of each parity) whose bits 2..3 differ between any two of
// 4 consecutive rows of one parity class.
template <int D> __device__ __forceinline__ int swz_b(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Per-lane byte offsets of the transposed operand reads (A = M^T over 16 rows of a
// staged tile, one 32-column block db): half h covers rows 4h .. 4h+3 of each 8-row
// group. The chunk swizzle depends on the row modulo 16 only, which a multiple of
// 16 rows does not change: one offset per (db, h), the 16-row step is a constant.
template <int D>
__device__ __forceinline__ uint32_t bwd_tr_off(int lane, int db, int h) {
  constexpr int CPR = D / 8;
  const int g16 = lane >> 4, t4 = (lane & 15) >> 2, u4 = lane & 3;
  const int row = (g16 >> 1) * 8 + t4 + 4 * h;
  const int ch = (4 * db + 2 * (g16 & 1) + (u4 >> 1)) ^ swz_b<D>(row);
  return (uint32_t)((row * CPR + ch) * 16 + (u4 & 1) * 8);
}

// Transposed operand of a staged tile: columns 32 db .. 32 db + 31, rows 16 st .. +15.
template <int D>
__device__ __forceinline__ u32x4_t bwd_tr_frag(const u32x4_t* tile, const uint32_t (&off)[D / 32][2],
                                               int db, int st) {
  constexpr int CPR = D / 8;
  const unsigned char* b = reinterpret_cast<const unsigned char*>(tile) + 16 * st * CPR * 16;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b + off[db][0]));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b + off[db][1]));
  const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
}

// Row operand of a staged tile (A = M over 32 rows, 16 columns): MFMA row m reads tile
// row r0 + key_of_row(m), columns 16 ds + 8 hh .. +7.
template <int D>
__device__ __forceinline__ u32x4_t bwd_row_frag(const u32x4_t* tile, int r0, int l32, int hh, int ds) {
  constexpr int CPR = D / 8;
  const int row = r0 + key_of_row(l32);
  return tile[row * CPR + ((2 * ds + hh) ^ swz_b<D>(row))];
}

// Store a transposed accumulator set (rows = head dims, lane = one output row `row`)
// times `mul` as 16-bit values into row `row` of a [N, D] matrix.
template <bool BF16, int D>
__device__ __forceinline__ void bwd_store_rows(uint16_t* dst, const f32x16_t (&acc)[D / 32], int row,
                                               int hh, float mul) {
  using E = Elt<BF16>;
  uint16_t* r = dst + (size_t)row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = db * 32 + g * 8 + hh * 4;
      const uint32_t w0 = E::pack(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul);
      const uint32_t w1 = E::pack(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
      *reinterpret_cast<u32x2_t*>(r + dcol) = u32x2_t{w0, w1};
    }
}

// ---- D = rowsum(dO * O): one pass, CPR threads per row ---------------------------------
// Written to p.delta (the dQ output's memory, as float32) for the dK/dV kernel, which
// would otherwise recompute it for every key tile, with L log2(e) next to it in p.lse2;
// the dQ kernel runs after it and computes D and reads L for its own rows.
template <bool BF16, int D>
__global__ void __launch_bounds__(256) fa_bwd_delta_kernel(const BwdParams p) {
  using E = Elt<BF16>;
  constexpr int CPR = D / 8, RPB = 256 / CPR;  // chunks per row, rows per workgroup
  const long long rows = (long long)p.BH * p.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CPR;
  const int ch = threadIdx.x % CPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4_t a = ld16(p.dout + row * D + ch * 8), b = ld16(p.o + row * D + ch * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = E::dot2(a[w], b[w], acc);
  }
#pragma unroll
  for (int m = 1; m < CPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (row < rows && ch == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * 1.4426950408889634f;
  }
}

// ---- dQ: one workgroup per 128 query rows -------------------------------------------
template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fa_bwd_dq_kernel(const BwdParams p) {
  using E = Elt<BF16>;
  constexpr int NW = 4, BQ = 128, BK = 64, CPR = D / 8, NDS = D / 16;
  __shared__ __attribute__((aligned(1024))) u32x4_t ks2[2][BK * CPR];
  __shared__ __attribute__((aligned(1024))) u32x4_t vs2[2][BK * CPR];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int N = p.N;
  const int n_qt = (N + BQ - 1) / BQ;
  int bh, rank;
  tile_order<CAUSAL>(blockIdx.x, p.BH, n_qt, bh, rank);
  const int qt = CAUSAL ? n_qt - 1 - rank : rank;  // the last query tile sees the most keys
  const size_t head = (size_t)bh * (size_t)N * D;
  const int q0 = qt * BQ, qi = q0 + wid * 32 + l32;
  const int qr = min(qi, N - 1);  // rows past N load row N-1 and are never stored
  const int n_kt = CAUSAL ? (min(q0 + BQ, N) + BK - 1) / BK : (N + BK - 1) / BK;
  const bool wave_live = q0 + wid * 32 < N;
  const int w_last = min(q0 + wid * 32 + 31, N - 1);
  const int lim = CAUSAL ? min(qi, N - 1) : N - 1;  // last key this lane's query sees

  // Q and dO as B operands (lane: query qi, columns 16 ds + 8 hh .. +7), D_i and L_i
  u32x4_t qf[NDS], dof[NDS];
  float dpart = 0.f;
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    const size_t off = head + (size_t)qr * D + ds * 16 + hh * 8;
    qf[ds] = ld16(p.q + off);
    dof[ds] = ld16(p.dout + off);
    const u32x4_t of = ld16(p.o + off);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dpart = E::dot2(dof[ds][w], of[w], dpart);
    }
  }
  const float Dq = xhalf_sum(dpart);
  const float L2 = p.lse[(size_t)bh * N + qr] * 1.4426950408889634f;

  f32x16_t dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;
  uint32_t troff[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) troff[db][h] = bwd_tr_off<D>(lane, db, h);

  // Key tiles: K and V go HBM -> LDS by buffer loads with an LDS destination into two
  // buffers (tile j in buffer j % 2; iteration j issues tile j+1 into the other one,
  // whose readers passed the previous barrier), one barrier per tile. Lane l of copy c
  // writes chunk (wid + NW c) * 64 + l and fetches the logical chunk the swizzle puts
  // there; the buffer range ends at key N, so keys past N read as zeros (masked).
  constexpr int TOT = BK * CPR, PERW = TOT / (64 * NW);
  static_assert(TOT % (64 * NW) == 0, "whole 1 KB copies per wave");
  const int wu = __builtin_amdgcn_readfirstlane(wid);  // LDS destination base: wave-uniform
  int doff[PERW];
#pragma unroll
  for (int c = 0; c < PERW; ++c) {
    const int f = (wid + NW * c) * 64 + lane, row = f / CPR, ph = f % CPR;
    doff[c] = row * D + (ph ^ swz_b<D>(row)) * 8;
  }
  auto issue = [&](int kb0, u32x4_t* kdst, u32x4_t* vdst) {
    const int bytes = min(N - kb0, BK) * D * 2;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.k + head + (size_t)kb0 * D), (short)0, bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.v + head + (size_t)kb0 * D), (short)0, bytes, kBufferWord3);
    // (the LDS destinations and offsets are arguments: a lambda that captured the shared
    // arrays or the offset array here made the host pass drop the kernel's launch stub)
    auto copy = [&](int c, int off) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kdst + (wu + NW * c) * 64), 16,
                                               off * 2, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vdst + (wu + NW * c) * 64), 16,
                                               off * 2, 0, 0, 0);
    };
#pragma unroll
    for (int c = 0; c < PERW; ++c) copy(c, doff[c]);
  };
  issue(0, ks2[0], vs2[0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int j = 0; j < n_kt; ++j) {
    const int k0 = j * BK, b = j & 1;
    if (j + 1 < n_kt) issue(k0 + BK, ks2[b ^ 1], vs2[b ^ 1]);
    const u32x4_t* ks = ks2[b];
    const u32x4_t* vs = vs2[b];
    if (wave_live && !(CAUSAL && k0 > w_last)) {  // every wave copies and meets the barrier
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      // S^T and dP^T of 32 keys x this wave's 32 queries
      f32x16_t st = {}, dpt = {};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        st = E::mfma(bwd_row_frag<D>(ks, 32 * kb, l32, hh, ds), qf[ds], st);
        dpt = E::mfma(bwd_row_frag<D>(vs, 32 * kb, l32, hh, ds), dof[ds], dpt);
      }
      // dS^T = P^T * (dP^T - D), P recomputed from L; register r holds key
      // k0 + 32 kb + 8 hh + rc(r), allowed when rc(r) <= t
      const int t = lim - (k0 + 32 * kb + 8 * hh);
      u32x4_t dsop[2];
      auto body = [&](bool masked) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float v2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int rc = key_of_reg(r + e, 0);
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r + e], p.c, -L2));
            if (masked && !(rc <= t)) pr = 0.f;
            v2[e] = pr * (dpt[r + e] - Dq);
          }
          dsop[r / 8][(r % 8) / 2] = E::pack(v2[0], v2[1]);
        }
      };
      // a register's key offset within its half is at most 23: when every lane allows
      // that much (tiles below the diagonal, away from the ragged end), no score is masked
      if (__builtin_amdgcn_ballot_w64(!(t >= 23)) == 0) body(false);
      else body(true);
      // dQ^T += K^T dS^T over these 32 keys (two 16-key steps)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dq[db] = E::mfma(bwd_tr_frag<D>(ks, troff, db, 2 * kb + s2), dsop[s2], dq[db]);
#if FA_BWD_DQ_SG
      // operand reads run FA_BWD_DQ_AHEAD products ahead: S^T and dP^T (one row read
      // each), then dQ (two transposed reads each); one ordered sequence over both
      // 32-key blocks
      __builtin_amdgcn_sched_group_barrier(0x100, FA_BWD_DQ_AHEAD, 0);
#pragma unroll
      for (int i = 0; i < 2 * NDS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + FA_BWD_DQ_AHEAD < 2 * NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * FA_BWD_DQ_AHEAD, 0);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + FA_BWD_DQ_AHEAD < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#endif
    }
    }  // live tile
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile j+1's copies
    __syncthreads();
  }
  if (wave_live && qi < N) bwd_store_rows<BF16, D>(p.dq + head, dq, qi, hh, p.scale);
}

// ---- dK, dV: one workgroup per 128 keys ----------------------------------------------
template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) fa_bwd_dkdv_kernel(const BwdParams p) {
  using E = Elt<BF16>;
  // Queries per staged tile: 128 rather than 64 halves the copies, barriers and loop
  // overhead per query (+2 to +7%).
  constexpr int BQ = 128;
  constexpr int NW = 4, BKV = 128, CPR = D / 8, NDS = D / 16;
  __shared__ __attribute__((aligned(1024))) u32x4_t qs2[2][BQ * CPR];
  __shared__ __attribute__((aligned(1024))) u32x4_t dos2[2][BQ * CPR];
  __shared__ __attribute__((aligned(16))) float lsh2[2][BQ];
  __shared__ __attribute__((aligned(16))) float dsh2[2][BQ];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, l32 = lane & 31, hh = lane >> 5;
  const int N = p.N;
  const int n_kt = (N + BKV - 1) / BKV;
  int bh, kt;
  tile_order<CAUSAL>(blockIdx.x, p.BH, n_kt, bh, kt);  // the first key tile sees the most queries
  const size_t head = (size_t)bh * (size_t)N * D;
  const int k0 = kt * BKV, kj = k0 + wid * 32 + l32;
  const bool wave_live = k0 + wid * 32 < N;
  const int n_qt = (N + BQ - 1) / BQ;
  const int i0 = CAUSAL ? k0 / BQ : 0;  // queries before k0 never see these keys

  // K and V of this wave's 32 keys as B operands (lane: key kj, columns 16 ds + 8 hh ..);
  // keys past N load row N - 1 and are masked
  u32x4_t kf[NDS], vf[NDS];
  {
    const int kr = min(kj, N - 1);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const size_t off = head + (size_t)kr * D + ds * 16 + hh * 8;
      kf[ds] = ld16(p.k + off);
      vf[ds] = ld16(p.v + off);
    }
  }

  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }
  uint32_t troff[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) troff[db][h] = bwd_tr_off<D>(lane, db, h);

  // Query tiles: Q and dO go HBM -> LDS by buffer loads with an LDS destination (no
  // register staging) into two buffers; L and D of the tile's rows (thread t < BQ: row
  // t; D from fa_bwd_delta_kernel) go through registers. Tile i lives in buffer i % 2:
  // iteration i issues tile i+1 into the other buffer, whose last readers (tile i-1)
  // passed the previous barrier, computes tile i, waits for its own copies, publishes
  // tile i+1's L and D, and meets one barrier. Each wave copies whole 1 KB pieces: lane
  // l of copy c writes chunk (wid + NW c) * 64 + l of the tile and fetches the logical
  // chunk the swizzle puts there. The buffer range ends at row N, so rows past N read as
  // zeros (their scores are masked); their L and D repeat row N - 1 (finite).
  constexpr int TOT = BQ * CPR, PERW = TOT / (64 * NW);
  static_assert(TOT % (64 * NW) == 0, "whole 1 KB copies per wave");
  const int wu = __builtin_amdgcn_readfirstlane(wid);  // LDS destination base: wave-uniform
  int doff[PERW];
#pragma unroll
  for (int c = 0; c < PERW; ++c) {
    const int f = (wid + NW * c) * 64 + lane, row = f / CPR, ph = f % CPR;
    doff[c] = row * D + (ph ^ swz_b<D>(row)) * 8;
  }
  float ln = 0.f, dn = 0.f;
  auto issue = [&](int qb0, u32x4_t* qdst, u32x4_t* ddst) {
    const int bytes = min(N - qb0, BQ) * D * 2;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.q + head + (size_t)qb0 * D), (short)0, bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.dout + head + (size_t)qb0 * D), (short)0, bytes, kBufferWord3);
    // (the LDS destinations and offsets are arguments: a lambda that captured the shared
    // arrays or the offset array here made the host pass drop the kernel's launch stub)
    auto copy = [&](int c, int off) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_t*)(qdst + (wu + NW * c) * 64), 16,
                                               off * 2, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t*)(ddst + (wu + NW * c) * 64), 16,
                                               off * 2, 0, 0, 0);
    };
#pragma unroll
    for (int c = 0; c < PERW; ++c) copy(c, doff[c]);
    if (tid < BQ) {
      const size_t r = (size_t)bh * N + min(qb0 + tid, N - 1);  // rows past N: masked
      ln = p.lse[r];
      dn = p.delta[r];
    }
  };
  auto publish = [&](float* lds_l, float* lds_d) {
    if (tid < BQ) {
      lds_d[tid] = dn;
      lds_l[tid] = ln * 1.4426950408889634f;
    }
  };
  issue(i0 * BQ, qs2[i0 & 1], dos2[i0 & 1]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  publish(lsh2[i0 & 1], dsh2[i0 & 1]);
  __syncthreads();
  for (int i = i0; i < n_qt; ++i) {
    const int qb0 = i * BQ, b = i & 1;
    if (i + 1 < n_qt) issue(qb0 + BQ, qs2[b ^ 1], dos2[b ^ 1]);
    const u32x4_t* qs = qs2[b];
    const u32x4_t* dos = dos2[b];
    const float* lsh = lsh2[b];
    const float* dsh = dsh2[b];
    if (wave_live) {  // every wave still copies its share and meets the barrier
    // Per 32-query block: S and dP (MFMA), the softmax terms (VALU), dV and dK (MFMA).
    // At d = 128 both blocks' S and dP are issued first, so block 1's products run while
    // block 0's softmax terms are computed, and block 1's softmax while block 0's dV, dK
    // run.
    auto sdp = [&](int qb, f32x16_t& s, f32x16_t& dp) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        s = E::mfma(bwd_row_frag<D>(qs, 32 * qb, l32, hh, ds), kf[ds], s);
        dp = E::mfma(bwd_row_frag<D>(dos, 32 * qb, l32, hh, ds), vf[ds], dp);
      }
    };
    // P and dS as 16-bit B operands. L and D of the rows: register r holds query
    // qb0 + 32 qb + 8 hh + rc(r), with rc(r) = (r & 7) + 16 (r >> 3); it sees this
    // lane's key when lo <= rc(r) < hi
    auto soft = [&](int qb, const f32x16_t& s, const f32x16_t& dp, u32x4_t (&pop)[2],
                    u32x4_t (&dsop)[2]) {
      f32x4_t lv[4], dv4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = 32 * qb + 16 * (g >> 1) + 8 * hh + 4 * (g & 1);
        lv[g] = *reinterpret_cast<const f32x4_t*>(lsh + ql);
        dv4[g] = *reinterpret_cast<const f32x4_t*>(dsh + ql);
      }
      const int base = qb0 + 32 * qb + 8 * hh;
      const int lo = CAUSAL ? kj - base : -32;
      const int hi = kj < N ? N - base : -32;
      auto body = [&](bool masked) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float pv[2], dv2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int re = r + e, rc = key_of_reg(re, 0);
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[re], p.c, -lv[re / 4][re % 4]));
            if (masked && !(rc >= lo && rc < hi)) pr = 0.f;
            pv[e] = pr;
            dv2[e] = pr * (dp[re] - dv4[re / 4][re % 4]);
          }
          pop[r / 8][(r % 8) / 2] = E::pack(pv[0], pv[1]);
          dsop[r / 8][(r % 8) / 2] = E::pack(dv2[0], dv2[1]);
        }
      };
      // every register r (rc(r) in [0, 32)) allowed in every lane: no per-score mask
      if (D == 128 && __builtin_amdgcn_ballot_w64(!(lo <= 0 && hi >= 32)) == 0) body(false);
      else body(true);
    };
    // dV^T += dO^T P and dK^T += Q^T dS over 32 queries (two 16-query steps)
    auto accum = [&](int qb, const u32x4_t (&pop)[2], const u32x4_t (&dsop)[2]) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = E::mfma(bwd_tr_frag<D>(dos, troff, db, 2 * qb + s2), pop[s2], dv[db]);
          dk[db] = E::mfma(bwd_tr_frag<D>(qs, troff, db, 2 * qb + s2), dsop[s2], dk[db]);
        }
    };
    static_assert(BQ % 64 == 0, "pairs of 32-query blocks per tile");
    if constexpr (D == 128 && FA_BWD_PIPE) {  // both blocks' S and dP of a pair first
      auto pair = [&](int q2) {
        f32x16_t s0, dp0, s1, dp1;
        u32x4_t pop0[2], dsop0[2], pop1[2], dsop1[2];
        sdp(q2, s0, dp0);
        sdp(q2 + 1, s1, dp1);
        soft(q2, s0, dp0, pop0, dsop0);
        accum(q2, pop0, dsop0);
        soft(q2 + 1, s1, dp1, pop1, dsop1);
        accum(q2 + 1, pop1, dsop1);
      };
      // unrolled, the non-causal tile spills registers (-1%); rolled it is 3-4% faster,
      // while the causal tile is 1% faster unrolled
      if constexpr (CAUSAL) {
#pragma unroll
        for (int q2 = 0; q2 < BQ / 32; q2 += 2) pair(q2);
      } else {
#pragma unroll 1
        for (int q2 = 0; q2 < BQ / 32; q2 += 2) pair(q2);
      }
    } else {  // d = 64 keeps two waves per SIMD with one block at a time
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        f32x16_t s, dp;
        u32x4_t pop[2], dsop[2];
        sdp(qb, s, dp);
        soft(qb, s, dp, pop, dsop);
        accum(qb, pop, dsop);
      }
    }
    }  // wave_live
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile i+1's copies, its L and D
    if (i + 1 < n_qt) publish(lsh2[b ^ 1], dsh2[b ^ 1]);
    __syncthreads();
  }
  if (wave_live && kj < N) {
    bwd_store_rows<BF16, D>(p.dk + head, dk, kj, hh, p.scale);
    bwd_store_rows<BF16, D>(p.dv + head, dv, kj, hh, 1.0f);
  }
}

// ---- launches ------------------------------------------------------------------------
constexpr int kBwdRows = 128;  // query rows per dQ workgroup = keys per dK/dV workgroup

// The slot-scheduled dK/dV and dQ kernels (fa_bwd_wide.hpp, included by the translation
// units of the head dims); they need a nonzero scale (their causal masks set scores to an
// infinity of the sign that gives P = 0).
template <bool BF16, int D, bool CAUSAL>
__global__ void fa_bwd_dkdv_wide_kernel(const BwdParams p);
template <bool BF16, int D, bool CAUSAL>
__global__ void fa_bwd_dq_wide_kernel(const BwdParams p);
// query blocks of 32 per wave in that dQ kernel at head dim 128. Two (each K, K^T or V
// operand read from LDS then serves two products, as in the forward's wide kernel) passed
// every backward test but measured +0.7% without the causal mask and -20% with it, where
// the compiler spilled registers to scratch inside the loop; so one.
#ifndef FA_BQ_QB128
#define FA_BQ_QB128 1
#endif
template <int D> constexpr int kDqBlocks = D == 128 ? FA_BQ_QB128 : 1;

// One backward call: three launches in stream order, D into dq's memory, dK and dV
// (reading D), then dQ (overwriting that memory; it computes D for its own rows).
// Explicitly instantiated per head dim in fa_bwd_d64.hip and fa_bwd_d128.hip, which
// are compiled with different code-generation options.
template <bool BF16, int D, bool CAUSAL>
hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  const int tiles = (p.N + kBwdRows - 1) / kBwdRows;
  const long long rows = static_cast<long long>(p.BH) * p.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((fa_bwd_delta_kernel<BF16, D>),
                     dim3(static_cast<unsigned>((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool wide = FA_BWD_WIDE && p.c != 0.f;
  if (wide)
    hipLaunchKernelGGL((fa_bwd_dkdv_wide_kernel<BF16, D, CAUSAL>), dim3(tiles * p.BH), dim3(256), 0,
                       s, p);
  else
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<BF16, D, CAUSAL>), dim3(tiles * p.BH), dim3(256), 0, s,
                       p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int qrows = 128 * kDqBlocks<D>;  // query rows per workgroup of that kernel
  if (wide)
    hipLaunchKernelGGL((fa_bwd_dq_wide_kernel<BF16, D, CAUSAL>),
                       dim3((p.N + qrows - 1) / qrows * p.BH), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((fa_bwd_dq_kernel<BF16, D, CAUSAL>), dim3(tiles * p.BH), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
