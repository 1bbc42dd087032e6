/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention-2 forward library.
 *
 * The operation: exact scaled-dot-product attention O = softmax(scale*Q K^T) V
 * per (batch, head), computed tile by tile with the online softmax (running
 * row max m, running denominator l, unnormalised fp32 accumulator; both l and
 * the accumulator rescaled by exp(m_old - m_new) on every key tile, a single
 * division at the end), so the N x N score matrix never exists in memory.
 * Defined on "A09 - Advanced Triton & FlashAttention" (section 3, The
 * rescaling update, written out, and The kernel, in pseudocode) and
 * "FlashAttention 2 from PyTorch to Triton" (What I am building: the FA2
 * forward and its row log-sum-exp output L = m + log l). The tensor contract
 * (contiguous [B, H, N, D], fp16/bf16, causal or not, head dim 64 or 128)
 * follows the scope of "Building a Verifiable FlashAttention Forward from
 * PyTorch to Triton"; an fp32 path is added as a precision check.
 *
 * Conventions shared by every entry point:
 *  - q, k, v, o are device pointers to contiguous row-major [B, H, N, D]
 *    tensors of element type `dtype`; o has the same type as the inputs.
 *    (fa_fwd_ex: q and o are [B, H, Nq, D], k and v are [B, H, Nk, D].)
 *  - lse is a device pointer to a contiguous fp32 [B, H, N] tensor ([B, H, Nq]
 *    for fa_fwd_ex), or NULL (then the log-sum-exp is not written). LSE uses
 *    the natural log.
 *  - causal != 0 applies the top-left causal mask: query i sees key j only
 *    when j <= i ("Building a Verifiable FlashAttention Forward", Part 1).
 *    fa_fwd_ex can align the mask bottom-right instead.
 *  - scale multiplies Q K^T; it must be finite and > 0 (the usual value is
 *    1/sqrt(D)).
 *  - Ownership: the caller owns every buffer; the library allocates no device
 *    memory and keeps no state between calls.
 *  - The call is asynchronous and stream-ordered on `stream` (a hipStream_t;
 *    NULL = the null stream). It returns after the kernel is enqueued; the
 *    outputs are valid once the caller has synchronised that stream. A fault
 *    on the device is reported by that synchronisation, not by the return.
 *  - o and lse must not overlap q, k, v or each other (checked on the host).
 *  - Error behaviour: every argument is validated before any HIP call. On an
 *    invalid argument nothing is launched and a negative code is returned;
 *    the outputs are left untouched. Thread-safe and reentrant.
 *  - Limits: 1 <= B, H, N (Nq, Nk); B*H*ceil(N/128) < 2^31 workgroups; one
 *    head's tensor (N*D*element size bytes) must be below 2^31 bytes;
 *    pointers must be 16-byte aligned.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_dtype { FA_DTYPE_FP32 = 0, FA_DTYPE_FP16 = 1, FA_DTYPE_BF16 = 2 };

/* Alignment of the causal mask when the query and key lengths differ. */
enum fa_causal_align {
  FA_CAUSAL_TOP_LEFT = 0,     /* query i sees keys j <= i                   */
  FA_CAUSAL_BOTTOM_RIGHT = 1  /* query i sees keys j <= i + (Nk - Nq)       */
};

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, size < 1, bad scale, overlap   */
  FA_ERR_UNSUPPORTED = -2, /* D not in {64, 128}, unknown dtype, too large */
  FA_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned              */
  FA_ERR_HIP = -4,         /* the HIP launch failed; see fa_strerror        */
  FA_ERR_SCRATCH = -5      /* fa_fwd_splitkv_noalloc: partials too large    */
};

/*
 * Attention forward for self-attention of length N: O [B,H,N,D] and, when
 * lse != NULL, LSE [B,H,N] = m + log(l) per row (natural log, fp32).
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale,
           int dtype, void *stream);

/*
 * Attention forward with separate query and key/value lengths (cross
 * attention): q, o [B,H,Nq,D]; k, v [B,H,Nk,D]; lse [B,H,Nq] or NULL. The
 * grid, the query-row mask, the store and LSE use Nq; the key loop, the K/V
 * loads and the score mask use Nk ("Triton: FlashAttention-2 Forward Pass",
 * Masks and sentinels, on cross-attention). With causal != 0, causal_align
 * selects the diagonal: FA_CAUSAL_TOP_LEFT (query i sees keys j <= i, the
 * convention "How to profile and optimise kernels", Round 4, attributes to
 * SDPA's is_causal) or FA_CAUSAL_BOTTOM_RIGHT (j <= i + Nk - Nq, which the
 * same passage attributes to the FlashAttention library since 2.1); it is
 * ignored when causal == 0 and must still be one of the two values. A query
 * row that sees no key (bottom-right with Nq > Nk: rows i < Nq - Nk) gets
 * O = 0 and LSE = -inf. Requires 1 <= Nq, 1 <= Nk; the other limits and the
 * error codes are those of fa_fwd (FA_ERR_INVALID_ARG also for an unknown
 * causal_align). fa_fwd(..., N, ...) equals fa_fwd_ex(..., N, N, ...).
 */
int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
              int causal, int causal_align, float scale, int dtype,
              void *stream);

/*
 * Split-KV forward: the same result as fa_fwd_ex, for grids too small to fill
 * the chip (few heads times query tiles, e.g. short query blocks). Each
 * (batch*head, 128-row query tile) is split into num_splits shares of its key
 * tiles; every share writes a normalised fp32 partial O_s and its row
 * log-sum-exp LSE_s into `workspace`, and a second kernel on the same stream
 * combines them as LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s
 * (the rebasing of "A09 - Advanced Triton & FlashAttention", section 3, across
 * key partitions; the pages name split-KV as the use of a consistent exponent
 * base in "Building a Verifiable FlashAttention Forward from PyTorch to
 * Triton", Part 3). Arguments as fa_fwd_ex, plus:
 *  - num_splits: 1 .. 32, or 0 to let the library choose
 *    (fa_splitkv_auto_splits). With one split the single-pass kernel runs
 *    and the workspace is not used (it may then be NULL).
 *  - workspace: device memory owned by the caller, 256-byte aligned, at least
 *    fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits) bytes, not
 *    overlapping any other argument. Its contents on entry do not matter;
 *    the library allocates nothing. Calls that share a workspace must be
 *    ordered (same stream, or synchronised).
 * Errors: those of fa_fwd_ex; FA_ERR_INVALID_ARG for num_splits outside
 * 0 .. 32, a NULL or too small workspace, or a workspace overlapping another
 * argument; FA_ERR_ALIGNMENT for a workspace not 256-byte aligned.
 */
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o,
                   float *lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                   int64_t D, int causal, int causal_align, float scale,
                   int dtype, int num_splits, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Split-KV forward that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation). The same computation and kernels as
 * fa_fwd_splitkv, with the same arguments minus the workspace: the fp32
 * partials live in a static device array inside the library,
 * FA_SPLITKV_SCRATCH_BYTES bytes, one copy per GPU, held from the first use
 * on that GPU until the process ends. Every call on one GPU reuses that
 * array, so calls that may overlap on one GPU (different streams without
 * ordering) race and must not be issued; calls ordered on one stream are
 * fine. Its contents on entry do not matter. The first call on a GPU looks
 * up the array's device address (no allocation).
 * Errors: those of fa_fwd_splitkv for the shared arguments, and
 * FA_ERR_SCRATCH, with nothing launched, when the partials for these sizes
 * and num_splits, fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits)
 * bytes, exceed FA_SPLITKV_SCRATCH_BYTES (every automatic split choice,
 * num_splits = 0, fits).
 */
#define FA_SPLITKV_SCRATCH_BYTES (32u << 20)
int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o,
                           float *lse, int64_t B, int64_t H, int64_t Nq,
                           int64_t Nk, int64_t D, int causal, int causal_align,
                           float scale, int dtype, int num_splits, void *stream);

/* Workspace bytes fa_fwd_splitkv needs for these sizes and num_splits (0 =
 * the library's choice); 0 when that is a single split, or for invalid sizes. */
size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq,
                                     int64_t Nk, int64_t D, int num_splits);

/* The number of splits fa_fwd_splitkv picks for num_splits = 0: 1 when the
 * single-pass grid (B*H*ceil(Nq/128) workgroups) exceeds 128; otherwise about
 * one workgroup per CU (256 / grid), limited so that each split keeps at
 * least 8 key tiles of 64 keys at D = 128 (16 at D = 64), and at most 32. */
int fa_splitkv_auto_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D);

/*
 * Backward pass: dQ, dK, dV of O = softmax(scale Q K^T) V for an upstream
 * gradient dout, from the forward's inputs, its output o and its row
 * log-sum-exp lse (natural log, as fa_fwd_ex writes it). The probabilities
 * are recomputed tile by tile as P = exp(S - L), the row vector
 * D = rowsum(dout * o) is formed first, the key gradients come from a kernel
 * that walks the query tiles of each key tile, and dQ from a second pass
 * (no atomics, deterministic): "FlashAttention 2 from PyTorch to Triton",
 * What is wrong with this kernel, item 5. With dS = P (dout V^T - D):
 * dV = P^T dout, dQ = scale dS K, dK = scale dS^T Q.
 *  - q, o, dout, dq: [B,H,Nq,D]; k, v, dk, dv: [B,H,Nk,D]; all of `dtype`,
 *    which must be FA_DTYPE_FP16 or FA_DTYPE_BF16 (FA_ERR_UNSUPPORTED for
 *    fp32). lse: fp32 [B,H,Nq], required.
 *  - delta: caller-owned fp32 [B,H,Nq] scratch; on return it holds D.
 *  - causal / causal_align / scale as in fa_fwd_ex (use the forward's).
 *  - Keys that no query sees get dK = dV = 0; query rows that see no key
 *    (lse = -inf) get dQ = 0.
 *  - dq, dk, dv and delta must not overlap each other or any input
 *    (FA_ERR_INVALID_ARG); every pointer must be 16-byte aligned.
 * Asynchronous on `stream` like the forward; allocates nothing.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const void *dout, const float *lse, void *dq, void *dk, void *dv,
           float *delta, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
           int64_t D, int causal, int causal_align, float scale, int dtype,
           void *stream);

/*
 * As fa_fwd, with only the first n_kv keys (0 <= n_kv <= N) visible: keys
 * j >= n_kv are masked for every query. The query and key lengths play
 * separate roles, as "Triton: FlashAttention-2 Forward Pass" (Masks and
 * sentinels) asks. With n_kv = 0 every row sees no key; such a row gets
 * O = 0 and LSE = -inf (the guard for fully masked rows of that page's
 * "The rescale direction"). fa_fwd(...) equals fa_fwd_nk(..., N, ...).
 */
int fa_fwd_nk(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t N, int64_t n_kv, int64_t D,
              int causal, float scale, int dtype, void *stream);

/*
 * Tuning entry: as fa_fwd_nk but runs kernel variant `variant` (0 = the
 * default choice of fa_fwd; 1 .. fa_num_variants()-1 = alternative tile
 * shapes / schedules of the same kernel family, all computing the same
 * result). FA_ERR_UNSUPPORTED if the variant does not exist for this
 * dtype and D.
 */
int fa_fwd_variant(const void *q, const void *k, const void *v, void *o,
                   float *lse, int64_t B, int64_t H, int64_t N, int64_t n_kv,
                   int64_t D, int causal, float scale, int dtype, void *stream,
                   int variant);

/* Number of variants (see fa_fwd_variant) and a short name for each;
 * the name of an unknown variant is "". */
int fa_num_variants(void);
const char *fa_variant_name(int variant);

/* Static text for a status code. For FA_ERR_HIP it is the HIP error string
 * of the most recent failure on the calling thread. Never NULL. */
const char *fa_strerror(int code);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
