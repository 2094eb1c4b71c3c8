// fa_common.hpp — types and helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N;          // sequence length
  int d;          // true head dim (row stride of q, k, v, o)
  int BH;         // B * H
  int n_qt;       // query tiles per head
  float c;        // |scale| * log2(e)
  uint32_t qsign; // 0x80008000 when scale < 0: Q is negated on load (exact), else 0
  float tau;      // rescale threshold in log2 units (fast kernel; 0: every tile)
  // split-KV partial pass: keys [s * split_keys, (s + 1) * split_keys) for split s; the
  // normalized partial O (float32) and partial L of split s go to o_part / l_part
  int split_keys;
  float* o_part;
  float* l_part;
};

// --- element type -----------------------------------------------------------------
template <bool BF16> struct Elt;
template <> struct Elt<true> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // round-to-nearest-even pack of two floats (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2_t x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
  }
  // acc + lo + hi of a packed pair (v_dot2c_f32_bf16 against (1, 1))
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
  }
  // acc + a.lo * b.lo + a.hi * b.hi of two packed pairs
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  }
};
template <> struct Elt<false> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  // round-to-nearest-even pack of two floats (v_cvt_pk_f16_f32)
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f32x2_t x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
  }
  // acc + lo + hi of a packed pair (v_dot2c_f32_f16 against (1, 1))
  static __device__ __forceinline__ float sum2(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w),
                                  __builtin_bit_cast(f16x2_t, 0x3c003c00u), acc, false);
  }
  // acc + a.lo * b.lo + a.hi * b.hi of two packed pairs
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  acc, false);
  }
};

// acc += A B with the accumulator held in AGPRs, for accumulators that only MFMAs touch
// until the end (the ones the VALU reads stay in VGPRs). Written out because the
// compiler picks one register file for all MFMA accumulators of a kernel. The compiler
// does not see these as matrix instructions: callers keep the sources of one step live
// until the next step is issued, and pad before the VALU reads the accumulator.
template <bool BF16>
__device__ __forceinline__ void mfma_acc_agpr(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  if (BF16)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Word 3 of a raw (stride 0) buffer resource on CDNA: 32-bit data format.
constexpr int kBufferWord3 = 0x00020000;

// XOR swizzles of the 16-byte chunks of LDS row `row` of a K tile and of a V tile
// (head dim D, rows of D/8 chunks). Both are permutations of a row's chunks, chosen
// so the operand reads of the fast kernels are bank-conflict free: 16 lanes reading
// one logical chunk of 16 different K rows hit 16 different bank quads, and the
// 4-row x 4-chunk transposed reads of V spread over distinct banks.
template <int D> __device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D> __device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Layout of an O tile staged in LDS on its way to HBM (rows of CPR 16-byte chunks, CPR
// = 8 or 16). The writers are lanes that each hold 8 bytes (one half, hh) of chunk c of
// row r, 32 rows per instruction; the readers take whole 16-byte chunks. Chunk c of row r
// sits at chunk o_pos(r, c), and its two halves trade places there when o_swap(r, c)
// is 1. Every 16 consecutive rows of one write then cover the 32 two-bank pairs of a
// 128-byte bank window once (and the 32 rows the 64 pairs of 256 bytes), and every 8
// (16) lanes of a read one row's chunks, so neither side conflicts on banks.
template <int CPR> __device__ __forceinline__ int o_pos(int r, int c) {
  return CPR == 16 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
}
template <int CPR> __device__ __forceinline__ int o_swap(int r, int c) {
  return CPR == 16 ? (((c ^ r) >> 3) ^ (r >> 4)) & 1 : (r ^ (r >> 4)) & 1;
}
// Byte offset in the staged tile of half hh of chunk c of row r.
template <int CPR> __device__ __forceinline__ int o_half_off(int r, int c, int hh) {
  return (r * CPR + o_pos<CPR>(r, c)) * 16 + ((hh ^ o_swap<CPR>(r, c)) << 3);
}
// Chunk c of row r read back from the staged tile in logical order.
template <int CPR>
__device__ __forceinline__ u32x4_t o_chunk_read(const unsigned char* t, int r, int c) {
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(t + (r * CPR + o_pos<CPR>(r, c)) * 16);
  return o_swap<CPR>(r, c) ? u32x4_t{x[2], x[3], x[0], x[1]} : x;
}

// Raw buffer resource over `bytes` bytes at address a (stride 0, 32-bit format): reads
// past the end return zeros.
__device__ __forceinline__ u32x4_t buffer_rsrc(uint64_t a, uint32_t bytes) {
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kBufferWord3};
}
// min(max(x, 0), hi) on the scalar unit, for a wave-uniform x (a clamp the compiler
// would do with v_med3 on the vector unit, leaving a buffer resource word in a vector
// register)
__device__ __forceinline__ uint32_t sclamp(int x, int hi /* a constant */) {
  uint32_t r;
  asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2" : "=&s"(r) : "s"(x), "n"(hi) : "scc");
  return r;
}

// HBM -> LDS copies issued as inline assembly, so the compiler's memory counter model
// does not see them and adds no waits of its own: the kernels order them with explicit
// vmcnt waits and barriers. They write no register. One copy: lane l's 16 (lds_copy16)
// or 4 (lds_copy4) bytes at byte offset voff of the buffer land at LDS address lds +
// lds_off + 16 l (or 4 l); M0 holds the LDS address, and bytes past the buffer's size
// read as 0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(u32x4_t rsrc, uint32_t voff, uint32_t lds,
                                           int lds_off /* a constant after unrolling */) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds), "n"(lds_off) : "m0", "scc");
}
__device__ __forceinline__ void lds_copy4(u32x4_t rsrc, uint32_t voff, uint32_t lds,
                                          int lds_off /* a constant after unrolling */) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds), "n"(lds_off) : "m0", "scc");
}
#pragma clang diagnostic pop

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// MFMA row m of the S^T product holds key rho(m) of the 32-key block: bits 2 and 3 swapped.
__device__ __forceinline__ int key_of_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// Key (within the 32-key block) held by accumulator register r of lane-half h.
__device__ __forceinline__ constexpr int key_of_reg(int r, int h) { return r + 8 * h + (r & 8); }
// Reductions across the two wave halves (lane l and lane l^32 hold the same query
// row): one v_permlane32_swap, which leaves {x[l], x[l^32]} in the two results of
// every lane, in the same order on both halves (so both halves get equal bits).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                   __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)pr[0]),
                         __builtin_bit_cast(float, (uint32_t)pr[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                   __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)pr[0]) + __builtin_bit_cast(float, (uint32_t)pr[1]);
}

// Workgroup -> (head, tile rank), for a grid of BH * n_t workgroups. Workgroups are
// dispatched round-robin over the 8 XCDs (bid % 8). When BH is a multiple of 8 all tiles
// of a head run on one XCD, so its rows are fetched into that XCD's L2 only. Under the
// causal mask ranks are issued in increasing order over all heads (rank 0 = the tile
// with the most work, which the caller maps to its tile index), so the short tiles fill
// the tail of the grid.
template <bool CAUSAL>
__device__ __forceinline__ void tile_order(int bid, int BH, int n_t, int& bh, int& rank) {
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, s = bid >> 3, hpx = BH >> 3;
    if (CAUSAL) {
      rank = s / hpx;
      bh = (s % hpx) * 8 + xcd;
    } else {
      bh = xcd * hpx + s / n_t;
      rank = s % n_t;
    }
  } else if (CAUSAL) {
    rank = bid / BH;
    bh = bid % BH;
  } else {
    bh = bid / n_t;
    rank = bid % n_t;
  }
}

// Forward kernels: the last query tile sees the most keys under the causal mask.
template <bool CAUSAL>
__device__ __forceinline__ void decode_tile(const Params& p, int bid, int& bh, int& qt) {
  int rank;
  tile_order<CAUSAL>(bid, p.BH, p.n_qt, bh, rank);
  qt = CAUSAL ? p.n_qt - 1 - rank : rank;
}

}  // namespace fa
