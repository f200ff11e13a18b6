/*
 * fa.h - C ABI of exact attention (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * What it computes. For every batch b and head h, with Q, K, V the [N, d]
 * slices of that (b, h):
 *
 *     S = scale * Q K^T              (N x N, never written to memory)
 *     S[i][j] = -inf  for j > i      (only when causal != 0)
 *     O = softmax_rows(S) V          (N x d)
 *     LSE[i] = log(sum_j exp(S[i][j]))   (natural log, one fp32 per query row)
 *
 * This is exact attention as defined on the page "Learn: The Memory Wall &
 * FlashAttention", section 4 "The attention memory problem", computed in one
 * fused kernel with the online-softmax recurrence of section 5.1 of the same
 * page (running max, running sum, rescaled unnormalised accumulator, one
 * division at the end) and the FA2 work split of "FlashAttention 2 & 3: Work
 * Partitioning, Warp Specialization & FP8" (sections "Edit 1" to "Edit 3").
 * LSE is the per-row logsumexp L = m + log l that the same page's section "The
 * backward pass" says the forward saves. The causal mask is top-left aligned:
 * query i sees keys 0..i (the mask of that page's reference loop).
 *
 * Conventions for every entry point:
 * - Tensors are dense, contiguous, row-major [B, H, N, d] ("BHND": batch, head,
 *   sequence, head dim); LSE is [B, H, N] fp32. Queries and keys have the same
 *   length N (fa_decode: Nq queries against Nk keys, with its own layout).
 * - Pointers are device pointers (HIP device memory) owned by the caller. The
 *   library never allocates, frees or copies host memory, and never
 *   synchronises: work is enqueued on `stream` (a hipStream_t passed as void*,
 *   NULL for the null stream) and the call returns once it is enqueued.
 * - Arguments are checked on the host before anything is launched; on an
 *   argument error nothing is launched and no output is written. No exception
 *   crosses the ABI. After a launch, a launch error is reported as
 *   FA_ERR_LAUNCH (the state of the outputs is then undefined).
 * - B, H or N equal to 0 is an empty problem: FA_OK, nothing is launched.
 *   N need not be a multiple of any tile size.
 * - NaN or infinite inputs are not trapped; they propagate into the outputs.
 * - All entry points are safe to call from several host threads on different
 *   streams; calls on one stream execute in order.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULLPTR = -1,   /* a required pointer is NULL */
    FA_ERR_ALIGN = -2,     /* a pointer is not 16-byte aligned */
    FA_ERR_SHAPE = -3,     /* B, H or N negative, B*H*N > 2^31 - 1, or N*d*4 > 2^31 - 1 (one
                              head's fp32 bytes must fit the 31-bit range of buffer offsets) */
    FA_ERR_HEADDIM = -4,   /* d is not 64, 128 or 256 */
    FA_ERR_DTYPE = -5,     /* dtype is not one of fa_dtype */
    FA_ERR_SCALE = -6,     /* scale is not finite and > 0 */
    FA_ERR_LAUNCH = -7,    /* the HIP runtime reported an error at launch */
    FA_ERR_ARG = -8,       /* any other invalid argument (e.g. causal not 0/1) */
    FA_ERR_SCRATCH = -9    /* fa_decode_noalloc: the problem needs more than its static scratch */
} fa_status;

typedef enum {
    FA_F32 = 0,   /* float32 Q, K, V and O; fp32 arithmetic throughout */
    FA_BF16 = 1   /* bfloat16 Q, K, V and O; bf16 MFMA products, fp32 accumulation and softmax */
} fa_dtype;

/*
 * fa_fwd - fused attention forward.
 *   q, k, v  [B, H, N, d] of `dtype` (input, not modified).
 *   o        [B, H, N, d] of `dtype` (output). Must not overlap the inputs.
 *   lse      [B, H, N] fp32 (output), natural-log logsumexp of each row of the
 *            scaled, masked scores; may be NULL to skip it.
 *   d        64, 128 or 256.  scale: finite, > 0 (usually 1/sqrt(d)).
 *   causal   0 or 1.   dtype: an fa_dtype value.
 * Returns FA_OK or an fa_status error code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_prep_fp8 - incoherent rotation and per-block E4M3 quantisation of one tensor.
 *
 * Sources: "FlashAttention 2 & 3" page, section "Incoherent processing: rotate
 * away the outliers" (x -> x M with M = (1/sqrt(d)) H D, H the Sylvester
 * Hadamard matrix, D a diagonal of +-1 signs) and the fake quantiser there
 * (scale = amax / 448, 1 when amax is 0); "FlashAttention-3: How Warp
 * Specialization ..." page, section 4 "Technique 3" (block-wise scales, e4m3
 * with magnitudes up to 448).
 *
 *   x      [B, H, N, d] fp32 (input).
 *   x8     [B, H, N, d] bytes (output): OCP E4M3 codes (bias 7, max 448, no
 *          infinities), rounded to nearest even, saturated at +-448.
 *   s      [B, H, ceil(N/64)] fp32 (output): one scale per block of 64 rows
 *          (sequence positions) of one (b, h) across all d columns; the last
 *          block of a ragged N covers the remaining rows. s = amax / 448 of the
 *          rotated block (1 when the block is all zero) and
 *          x8 = e4m3(x_rotated / s), the division done in fp32.
 *   signs  [d] fp32 of +1/-1 (input), the diagonal D; NULL skips the rotation
 *          (plain block quantisation, e.g. for V).
 * The rotation is computed in fp64 with a fast Walsh-Hadamard transform and
 * rounded once to fp32 (the float64 product x M of the definition, rounded).
 */
int fa_prep_fp8(const float* x, void* x8, float* s, const float* signs,
                int B, int H, int N, int d, void* stream);

/*
 * fa_fwd_fp8 - fused attention forward on E4M3 inputs with per-block scales.
 *
 * Source: "FlashAttention-3: How Warp Specialization ..." page, section 4:
 * the score tile is s_Q * s_K * (Q8 K8^T) with FP32 accumulation, and the
 * softmax statistics and the output accumulator stay in high precision
 * ("FlashAttention 2 & 3" page, section "What stays in higher precision").
 * The pages also convert P to FP8 for the second product; this library keeps
 * P (and V, expanded exactly from E4M3) in fp16 for it and writes O in fp32:
 * inputs with outliers put values of magnitude up to ~70 into O, where an E4M3
 * or bf16 P, or a bf16 O, alone costs more than 6e-2 of output error.
 *
 *   q8, k8, v8  [B, H, N, d] E4M3 codes (as written by fa_prep_fp8; Q and K
 *               rotated with the same signs, V usually not rotated).
 *   sq, sk, sv  [B, H, ceil(N/64)] fp32 block scales of q8, k8, v8.
 *   o           [B, H, N, d] fp32 (output) = the attention of the
 *               dequantised inputs (if V was rotated, O is in the rotated basis).
 *   lse         [B, H, N] fp32 (output) or NULL, as in fa_fwd.
 *   d           64, 128 or 256.  scale, causal: as in fa_fwd.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8,
               const float* sq, const float* sk, const float* sv,
               void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream);

/*
 * fa_bwd - attention backward: the gradients of O = softmax(scale Q K^T [causal]) V.
 *
 * Source: "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8",
 * section "The backward pass: recompute, and the one identity that makes it
 * tile-able": P = exp(S - L) is rebuilt from the forward's logsumexp,
 * dV = P^T dO, dP = dO V^T, D = rowsum(dO o O), dS = P o (dP - D),
 * dQ = scale dS K, dK = scale dS^T Q. Three kernels on `stream`: D, then dK and dV
 * (parallel over key blocks), then dQ (parallel over query blocks; no atomics,
 * the result is deterministic).
 *
 *   q, k, v     [B, H, N, d] bfloat16, the forward's inputs.
 *   o           [B, H, N, d] bfloat16, the forward's output.
 *   dout        [B, H, N, d] bfloat16, the gradient of the loss with respect to o.
 *   lse         [B, H, N] fp32, the forward's logsumexp (fa_fwd's lse).
 *   dq, dk, dv  [B, H, N, d] bfloat16 (outputs). Must not overlap the inputs.
 *   delta       [2, B, H, N] fp32 workspace owned by the caller (receives -D, then
 *               -LSE log2(e), the exponent bias the key-parallel passes read).
 *   d           64 or 128 (others: FA_ERR_HEADDIM).  dtype: FA_BF16 only
 *               (others: FA_ERR_DTYPE).  scale, causal: as in the forward call.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_ext - the attention forward with grouped key/value heads, a sliding window and
 * packed variable-length sequences (any combination).
 *
 * Sources: the flash_attn interface example and its packed-batch example on "Learn: The
 * Memory Wall & FlashAttention"; Exercise 5 of "FlashAttention 2 & 3: Work Partitioning,
 * Warp Specialization & FP8" (sliding window with key blocks outside the window skipped
 * and the partial blocks masked).
 *
 * - Grouped heads: Hkv divides Hq; query head h reads key/value head h / (Hq / Hkv).
 * - Window: query i sees key j iff i - window_left <= j <= i + window_right; a negative
 *   bound means no limit on that side. With causal = 1 keys after the query are hidden
 *   as well (window_right is then irrelevant): (4095, 0) with causal is a window of
 *   4096 keys including the query. Key blocks outside every query's window are skipped.
 * - Packed sequences: with cu_seqlens == NULL the tensors are q, o [B, Hq, N, d],
 *   k, v [B, Hkv, N, d], lse [B, Hq, N] (bfloat16; lse fp32, optional). With cu_seqlens
 *   (device int32 [B + 1], 4-byte aligned: B sequences, sequence s is tokens
 *   cu_seqlens[s] .. cu_seqlens[s+1]-1, cu_seqlens[0] = 0, cu_seqlens[B] = N) the batch
 *   dimension is 1: q, o [Hq, N, d], k, v [Hkv, N, d], lse [Hq, N]; a query sees keys of
 *   its own sequence only, and window and causal positions count from the sequence start.
 *   max_seqlen (<= N) must be at least the longest sequence: rows beyond it are not
 *   written. The offsets are read on the GPU and clamped to [0, N]; offsets that
 *   decrease or exceed N give undefined outputs but no access outside the tensors.
 *   Tokens not covered by any sequence are not written.
 *
 *   d 64 or 128 (FA_ERR_HEADDIM); dtype FA_BF16 only (FA_ERR_DTYPE); Hkv < 1 or not a
 *   divisor of Hq, or max_seqlen outside [0, N] with cu_seqlens: FA_ERR_SHAPE.
 */
int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int N, int d, float scale, int causal,
               int window_left, int window_right, const int* cu_seqlens, int max_seqlen,
               int dtype, void* stream);

/*
 * fa_decode - attention of a few query positions against a long key/value
 * sequence (autoregressive decoding), split over the keys.
 *
 * Source: "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8",
 * the paragraph on the decode regime (FlashDecoding): the key/value sequence is
 * split across the compute units, each part computes a partial softmax state
 * (m, l, O~) and the parts are merged with the online-softmax combine of
 * "FlashAttention-3 & GPU Kernel Optimization", section "Online softmax tiling
 * mathematics". Grouped-query attention as in the flash_attn example of "Learn:
 * The Memory Wall & FlashAttention": Hkv divides Hq and query head h reads
 * key/value head h / (Hq / Hkv); the query heads of one group are computed
 * together, so K and V are read once per group.
 *
 *   q         [B, Hq, Nq, d] bfloat16: the last Nq positions of each sequence.
 *   k, v      [B, Hkv, Nk, d] bfloat16 (the key/value cache), Nq <= Nk.
 *   o         [B, Hq, Nq, d] bfloat16 (output).
 *   lse       [B, Hq, Nq] fp32 natural-log logsumexp (output), or NULL.
 *   causal    0: every query sees all Nk keys. 1: query i (0-based among the Nq)
 *             sees keys j <= Nk - Nq + i, the forward's mask when Nq = Nk.
 *   workspace fp32 scratch owned by the caller, at least
 *             fa_decode_workspace_size(...) bytes, 16-byte aligned; may be NULL
 *             when that size is 0. Its contents are overwritten; calls that share
 *             one workspace must not overlap in time.
 *   d 64 or 128 (others: FA_ERR_HEADDIM); dtype FA_BF16 only (FA_ERR_DTYPE);
 *   Hkv < 1, Hq not a multiple of Hkv, Nq > Nk: FA_ERR_SHAPE; workspace_bytes
 *   below the required size: FA_ERR_ARG.
 */
size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d);
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc - fa_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, kernels and results as fa_decode (bit for bit); it calls
 * no hipMalloc, hipFree or other allocating routine.
 *
 * The split states live in a static device array of the library (8,486,400 bytes, one copy
 * per GPU, held until the process ends): the largest workspace fa_decode_workspace_size gives
 * for any shape, so no shape is refused today; a shape that needed more would return
 * FA_ERR_SCRATCH before any launch. The first call on a GPU looks up that GPU's copy (the GPU
 * of `stream`, the current one for the null stream). Every call on one GPU shares its copy:
 * calls that overlap in time on one GPU (several streams, several host threads) race and give
 * undefined outputs; calls on one stream are ordered and safe. No contents need clearing
 * between calls (every state is written before it is read).
 */
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int dtype, void* stream);

/* fa_status_string - static, human-readable text for a status code (never NULL). */
const char* fa_status_string(int status);

/* fa_version - library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
