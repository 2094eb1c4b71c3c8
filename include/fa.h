/*
 * fa.h — C ABI of the FA2-order attention forward pass, and of its backward
 * pass, for AMD MI355X (gfx950).
 *
 * Sources for the operation (web pages on FlashAttention):
 *  [P1] currybab.bearblog.dev, "Triton으로 FlashAttention 구현하기 전에 -
 *       FA1, 2 forward pass"
 *  [P2] iq-universe.github.io, "FlashAttention은 어떻게 O(N²) 메모리 벽을 넘었나"
 *  [P3] ariser.io, "FlashAttention: 어텐션을 빠르게 만든 건 계산량보다 데이터
 *       이동이었다"
 * [P2] sections are cited by their heading, e.g. [P2] "FlashAttention: SRAM tiling으로
 * O(N²) HBM을 우회하다".
 *
 * The library never allocates device memory, keeps no pointer after a call returns
 * and needs no workspace except where an entry point takes one from the caller (the O(N)
 * extra memory of the [P1] "정리" comparison table is the L output itself); the one
 * exception, fa_fwd_splitkv_static, uses a fixed device array of its own. Its only
 * other global state is the compute-unit count and the LDS size per compute unit of each
 * device, read once per device (std::call_once) and immutable afterwards; they only
 * steer how many 8-bit workgroups share a compute unit (a performance hint, never a
 * correctness input). Calls are reentrant and thread-safe (fa_fwd_splitkv_static: see its
 * comment). No C++ exception crosses this boundary.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                                 */
  FA_ERR_SHAPE = -2,       /* B, H, N or d < 1; scale not finite; sizes overflow          */
  FA_ERR_UNSUPPORTED = -3, /* d > 128, or an unknown dtype code                           */
  FA_ERR_ALIAS = -4,       /* o or lse overlaps q, k, v, or each other                    */
  FA_ERR_ALIGN = -5,       /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned   */
  FA_ERR_HIP = -6,         /* the HIP runtime refused the launch; see fa_last_hip_error() */
  FA_ERR_SCRATCH = -7      /* fa_fwd_splitkv_static: partials exceed the static scratch   */
};

/* dtype codes for fa_fwd_ex() and fa_fwd_supported(). */
enum fa_dtype { FA_DTYPE_BF16 = 0, FA_DTYPE_FP16 = 1 };

/* Rescale threshold of fa_fwd / fa_fwd_fp16, and the largest one fa_fwd_ex accepts
 * (log2 units; see fa_fwd_ex). */
#define FA_DEFAULT_RESCALE_LOG2 8.0f
#define FA_MAX_RESCALE_LOG2 15.0f

/* Largest split count fa_fwd_splitkv accepts. */
#define FA_MAX_SPLITS 64

/* Bytes of the device-resident scratch array behind fa_fwd_splitkv_static (64 MiB). */
#define FA_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * fa_fwd — exact attention forward in the FA2 loop order, bfloat16 tensors.
 *
 * Computes, for every batch b < B, head h < H and query row i < N
 * ([P1] "왜 필요한가" problem statement; [P2] tiling pseudocode and
 * [P3] "N×N 행렬은 꼭 저장해야 할까" for the 1/sqrt(d)-style scale):
 *
 *   S_ij   = scale * sum_c Q[b,h,i,c] * K[b,h,j,c]      over allowed keys j
 *   P_ij   = exp(S_ij) / sum_j' exp(S_ij')                ([P1] softmax equation)
 *   O[b,h,i,:] = sum_j P_ij * V[b,h,j,:]
 *   lse[b,h,i] = log sum_j exp(S_ij)                       ([P1] FA2 section,
 *                                                           epilogue equation L = m + log l)
 *
 * A key j is allowed when j < N and, if causal != 0, j <= i (the lower-
 * triangular mask of [P2] "v2와 v3", under which whole key blocks above the
 * diagonal are skipped). lse is the natural logarithm of the scaled, masked
 * scores, so that exp(S_ij - lse_i) = P_ij as in the [P1] LSE identity.
 *
 * The work follows the [P1] FA2 section: the query row block is the outer
 * loop and key/value blocks the inner loop; each row keeps a running max m
 * and sum l on chip, rescales its unnormalised output by exp(m_old - m_new)
 * only, and divides by l once at the end. S and P never reach device memory.
 *
 * Arguments
 *   q, k, v  device pointers to contiguous row-major [B, H, N, d] bfloat16
 *            tensors (read only; they may alias each other). 16-byte aligned.
 *   o        device pointer to a contiguous row-major [B, H, N, d] bfloat16
 *            output, written with round-to-nearest-even. 16-byte aligned.
 *   lse      device pointer to a contiguous [B, H, N] float32 output. 4-byte aligned.
 *   B, H, N  batch, heads and sequence length (queries and keys), each >= 1.
 *   d        head dimension, 1 <= d <= 128. d = 64 and d = 128 take the fast
 *            path; any other d takes a bounds-checked path with zero-filled
 *            columns (same results, slower).
 *   scale    multiplier of the dot products; any finite value (the usual
 *            choice is 1/sqrt(d)).
 *   causal   0 for full attention, nonzero for the causal mask above.
 *   stream   a hipStream_t passed as void*; NULL means the default stream.
 *
 * Ownership: the caller allocates and frees all five buffers; o and lse must
 * not overlap q, k, v or each other. Totals must satisfy N*d < 2^31 and
 * B*H*N*d*2 bytes < 2^62.
 *
 * Errors: all validation happens on the host before any HIP call, so an
 * invalid call touches no device state and returns one of FA_ERR_NULL,
 * FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIAS or FA_ERR_ALIGN. A launch the
 * runtime refuses returns FA_ERR_HIP and records the hipError_t for
 * fa_last_hip_error() on the calling thread.
 *
 * Asynchrony: the call only enqueues the kernel on `stream` and returns;
 * faults inside the kernel surface at the caller's next synchronisation.
 * Non-finite inputs give unspecified (non-finite) outputs.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_fwd_fp16 — the same operation, arguments and contract as fa_fwd, for
 * IEEE float16 q, k, v and o (lse stays float32).
 */
int fa_fwd_fp16(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_fwd_ex — fa_fwd / fa_fwd_fp16 with the dtype as an argument (FA_DTYPE_BF16 or
 * FA_DTYPE_FP16; anything else returns FA_ERR_UNSUPPORTED) and an explicit rescale
 * threshold.
 *
 * The running-max update of the [P1] FA2 section (m_new = max(m_old, rowmax S),
 * alpha = exp(m_old - m_new) applied to l and the unnormalised O) is taken on a key
 * block only when some row's block max exceeds its current reference by more than
 * rescale_log2 (in log2 units, i.e. a factor 2^rescale_log2); otherwise the row
 * keeps the old reference and that block's probabilities may reach 2^rescale_log2.
 * The softmax is unchanged by the choice of reference (the max shift cancels, as the
 * [P1] "Online Softmax 개념" block form shows), so O and lse are the same up to
 * rounding for every threshold. rescale_log2 = 0 is the literal per-block update of
 * the pages. 0 <= rescale_log2 <= FA_MAX_RESCALE_LOG2 (which keeps float16
 * probabilities finite), else FA_ERR_SHAPE. fa_fwd and fa_fwd_fp16 use
 * FA_DEFAULT_RESCALE_LOG2. Head dims other than 64 and 128, and scale = 0, always
 * take the per-block update.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              float rescale_log2, void* stream);

/*
 * fa_fwd_fp8 — the operation of fa_fwd on 8-bit inputs: q, k, v hold OCP FP8 E4M3
 * codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F/0xFF NaN, no
 * infinity) with one float scale per tensor, so Q = q_scale * decode(q), and likewise for
 * K and V. Computes O = softmax(scale * Q K^T [+ causal mask]) V and L exactly as fa_fwd
 * defines them, on the decoded tensors, with 8-bit matrix products: the FP8 path of [P2]
 * "v2와 v3" (FP8 doubling the matrix throughput of 16-bit inputs).
 *
 * Numerics: Q K^T accumulates the 8-bit products in float32; the online softmax runs
 * in float32; the unnormalised probabilities are rounded to E4M3 (round to nearest
 * even, 3 mantissa bits) for the P V product, which makes O differ from the exact
 * result by up to a few 2^-4 relative errors of each probability (L does not see that
 * rounding). O is written as bfloat16 (RNE), L as float32.
 *
 * Arguments: q, k, v device pointers to contiguous row-major [B, H, N, d] byte tensors,
 * 16-byte aligned; o a bfloat16 [B, H, N, d] output, 16-byte aligned; lse float32
 * [B, H, N]. d must be 64 or 128 (FA_ERR_UNSUPPORTED). scale and the three tensor scales
 * must be finite and scale * q_scale * k_scale nonzero (FA_ERR_SHAPE). Ownership,
 * aliasing (o, lse may not overlap the inputs or each other), errors and asynchrony as
 * fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_scale, float k_scale,
               float v_scale, void* o, float* lse, int B, int H, int N, int d, float scale,
               int causal, void* stream);

/*
 * fa_fwd_splitkv — the operation of fa_fwd_ex (same outputs, up to rounding), with the
 * keys of every head split into ranges that separate workgroups process, for shapes
 * whose B * H * ceil(N / 128) query tiles are too few to fill the GPU (few heads,
 * moderate N).
 *
 * Each split runs the FA2-order forward over its key range and leaves its normalized
 * partial output O_s and partial logsumexp L_s (float32) in the workspace; a second
 * kernel merges them per row as L = log sum_s exp(L_s), O = sum_s exp(L_s - L) O_s,
 * the block merge of the online softmax ([P1] "Online Softmax 개념"; [P3]
 * "소프트맥스는 나누어 계산할 수 있다", the [1,2,3,4] example split into two blocks
 * of two).
 *
 * n_splits in [1, FA_MAX_SPLITS] is an upper bound: the keys per split are
 * ceil(N / n_splits) rounded up to a multiple of the query tile (256 rows at d = 128,
 * 128 at d = 64), so fewer splits may run. Under the causal mask a split that lies
 * wholly after a query tile contributes L_s = -inf.
 * d must be 64 or 128 (FA_ERR_UNSUPPORTED) and scale nonzero (FA_ERR_SHAPE).
 *
 * workspace: device memory of at least fa_fwd_splitkv_workspace_size(B, H, N, d,
 * n_splits) bytes, 256-byte aligned, overlapping no tensor argument; owned by the
 * caller, contents on entry ignored and on return unspecified. Concurrent calls need
 * distinct workspaces. Other arguments, ownership, errors and asynchrony as fa_fwd_ex
 * (dtype FA_DTYPE_BF16 / FA_DTYPE_FP16; the rescale threshold is the default).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   float scale, int causal, int n_splits, int dtype, void* stream);

/* Bytes of workspace fa_fwd_splitkv needs for these sizes; 0 when they are invalid
 * (B, H, N < 1, d not 64 or 128, n_splits outside [1, FA_MAX_SPLITS]). Host only. */
size_t fa_fwd_splitkv_workspace_size(int B, int H, int N, int d, int n_splits);

/*
 * fa_fwd_splitkv_static — fa_fwd_splitkv without the workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation. It allocates nothing: the float32 partials live
 * in a file-scope device array of FA_STATIC_SCRATCH_BYTES bytes that each GPU the
 * library runs on holds from the library's first use on that GPU until the process
 * ends. The array's device address is looked up once per device (hipGetSymbolAddress,
 * with that device current) on the first call on the device; that lookup failing
 * returns FA_ERR_HIP.
 *
 * Same operation, arguments, validation and asynchrony as fa_fwd_splitkv with the
 * caller's workspace replaced by that array. A call whose partials
 * (fa_fwd_splitkv_workspace_size(B, H, N, d, n_splits) bytes) exceed
 * FA_STATIC_SCRATCH_BYTES returns FA_ERR_SCRATCH before any HIP call. The partial pass
 * writes every partial the merge reads, so nothing needs clearing between calls.
 *
 * Every call on one GPU shares that GPU's array and leaves its partials there: calls
 * that overlap in time on one GPU (on different streams, or from several threads without
 * ordering) race on it and give unspecified results. Calls ordered on one stream are
 * safe.
 */
int fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, int n_splits,
                          int dtype, void* stream);

/*
 * fa_fwd_fa1 — the same outputs as fa_fwd_ex (up to rounding), computed in the FA1
 * loop order as an ablation of the FA2 order of fa_fwd ([P1] "FlashAttention 1
 * forward pass 알고리즘 분석" and the "정리" table): one workgroup per (batch, head)
 * walks the key/value blocks in the outer loop and all query blocks in the inner loop,
 * merging each block into the running m_i, l_i and normalized O_i with the alpha/beta
 * update and writing them back to device memory after every key block. Q is read
 * T_c = ceil(N / 64) times and O_i round-trips through memory, which is what the
 * table's HBM column counts; it is slow on purpose (B * H workgroups only).
 *
 * workspace: at least fa_fwd_fa1_workspace_size(B, H, N, d) bytes (float32 O_i, m_i,
 * l_i), 256-byte aligned, overlapping no tensor argument; caller-owned, contents on
 * entry ignored. d must be 64 or 128 and scale nonzero. Other arguments, errors and
 * asynchrony as fa_fwd_ex.
 */
int fa_fwd_fa1(const void* q, const void* k, const void* v, void* o, float* lse,
               void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
               float scale, int causal, int dtype, void* stream);

/* Bytes of workspace fa_fwd_fa1 needs; 0 for invalid sizes. Host only. */
size_t fa_fwd_fa1_workspace_size(int B, int H, int N, int d);

/*
 * fa_bwd — gradients of the attention of fa_fwd with respect to q, k and v,
 * bfloat16 tensors.
 *
 * For the loss sum_{b,h,i,c} O[b,h,i,c] * dO[b,h,i,c] (so dout is dLoss/dO), per
 * batch and head, with P the softmax of fa_fwd over the allowed keys:
 *
 *   dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO[i,c] * O[i,c],
 *   dS = P * (dP - D)   (elementwise, D broadcast along each row),
 *   dQ = scale * dS K,   dK = scale * dS^T Q.
 *
 * P is not stored by the forward pass: it is recomputed block by block as
 * P_ij = exp(S_ij - lse_i) ([P1] FA2 section, the LSE identity; [P2] "FlashAttention:
 * SRAM tiling으로 O(N²) HBM을 우회하다", the paragraph on recomputation in the backward
 * pass; [P3] "계산을 다시 하는 편이 싸다는 역설", which
 * trades that recomputation for the N x N matrix's HBM traffic). D_i equals
 * rowsum(P * dP) (the softmax Jacobian), computed from dO and O.
 *
 * Arguments
 *   q, k, v  the inputs of the forward call: [B, H, N, d] bfloat16, row-major,
 *            contiguous, 16-byte aligned (read only; they may alias each other).
 *   o, lse   fa_fwd's outputs for q, k, v with the same scale and causal
 *            ([B, H, N, d] bfloat16 and [B, H, N] float32; read only). Other
 *            values give the gradients of a different function (unspecified).
 *   dout     dLoss/dO, [B, H, N, d] bfloat16 (read only), 16-byte aligned.
 *   dq, dk, dv  outputs, [B, H, N, d] bfloat16, written with round-to-nearest-
 *            even; 16-byte aligned; each element written by exactly one workgroup.
 *            Between the call's kernels dq's memory also holds D (B*H*N float32):
 *            computed once there before the dK/dV kernel reads it, then overwritten
 *            by dQ, so on completion dq holds dQ. Nothing else is written.
 *   B, H, N  each >= 1.
 *   d        64 or 128 (FA_ERR_UNSUPPORTED otherwise).
 *   scale, causal  as passed to fa_fwd.
 *   stream   a hipStream_t passed as void*; NULL means the default stream.
 *
 * Ownership: the caller allocates and frees every buffer; no workspace is used.
 * dq, dk and dv may overlap neither each other nor any input. Size limits are
 * those of fa_fwd.
 *
 * Errors and asynchrony: as fa_fwd (validation on the host before any HIP call;
 * FA_ERR_HIP with fa_last_hip_error() when a launch is refused; the call only
 * enqueues three kernels on `stream`, in order: D, then dK and dV, then dQ).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, void* stream);

/*
 * fa_bwd_fp16 — the same operation, arguments and contract as fa_bwd, for IEEE
 * float16 q, k, v, o, dout, dq, dk, dv (lse stays float32).
 */
int fa_bwd_fp16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, void* stream);

/*
 * fa_fwd_supported — 1 if a call with this head dimension, dtype code
 * (FA_DTYPE_BF16 / FA_DTYPE_FP16) and mask (causal 0/1) is supported, else 0.
 * The support question is the one [P3] "실제로 적용한다면 먼저 재볼 것"
 * asks before adopting an implementation (dtype, head dim, mask). Pure host
 * function; never touches the device.
 */
int fa_fwd_supported(int d, int dtype, int causal);

/*
 * fa_device_supported — 1 if HIP device `device` is one this library has code for
 * (a gfx950 GPU, e.g. MI355X), else 0 (also when the device does not exist or the HIP
 * runtime reports an error). The GPU half of the support question of [P3] "실제로
 * 적용한다면 먼저 재볼 것". Reads the device properties; launches nothing.
 */
int fa_device_supported(int device);

/*
 * fa_device_info — compute-unit count and peak engine clock (kHz) of HIP device
 * `device`, as the runtime reports them (hipDeviceProp_t multiProcessorCount and
 * clockRate), so a caller can price a measured rate against the matrix-core peak of
 * that device: CUs x clock x 4096 flops per cycle for 16-bit MFMA on gfx950 (four
 * SIMDs, each finishing a 32x32x16 product, 32768 flops, every 32 cycles).
 * Returns FA_OK, FA_ERR_NULL for a NULL output pointer, or FA_ERR_HIP (no such device,
 * or the runtime failed; fa_last_hip_error() names it). Outputs are 0 on error.
 * Launches nothing.
 */
int fa_device_info(int device, int* cu_count, int* clock_khz);

/* Human-readable text of a status code (static storage; never NULL). */
const char* fa_strerror(int status);

/* The hipError_t (as int) behind the last FA_ERR_HIP on this thread, else 0. */
int fa_last_hip_error(void);

/* Library version string (static storage). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
