/*
 * fa2.h -- C ABI of the FlashAttention-2 forward pass, and its backward pass,
 * for AMD MI355X (gfx950).
 *
 * The operation is exact scaled-dot-product attention of one head, for every
 * (batch, head) pair:
 *
 *     O   = softmax(scale * Q K^T) V            (row-wise softmax)
 *     LSE = m + ln(l),  m = max_j s_ij,  l = sum_j exp(s_ij - m)
 *
 * Definitions: "3.6 Attention I -- the memory problem and FlashAttention
 * principles", sections 3.6.2 (scaled dot-product attention), 3.6.4 (stable
 * softmax and the online recurrence) and 3.6.7 (the row statistic
 * L = m + log l kept for the backward pass); "FlashAttention-2 from scratch
 * in CuTe", kernel-structure section (P = Q K^T / sqrt(d_h), fp16 inputs,
 * fp32 accumulation).  The causal option masks future keys as in 3.6.6 of
 * the first page.  The N x N score matrix is never written to memory: the
 * kernel walks key/value tiles with the online-softmax recurrence and
 * normalises once at the end.
 *
 * All functions are plain C, thread-safe and re-entrant; the library keeps no
 * state between calls and allocates no device memory (the backward pass
 * takes its one workspace, delta, from the caller) -- except the fixed
 * scratch buffer of fa2_fwd_splitkv_noalloc, one per GPU, whose calls on one
 * GPU must not overlap.
 */
#ifndef FA2_H_
#define FA2_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by fa2_fwd and fa2_bwd. */
typedef enum {
    FA2_OK = 0,
    FA2_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, grid too large,
                                non-finite or too large scale, output aliasing */
    FA2_ERR_UNSUPPORTED = 2, /* head dim not one of 32, 64, 96, 128, 256
                                (fa2_bwd: 32, 64, 96, 128)                     */
    FA2_ERR_MISALIGNED = 3,  /* a pointer not 16-byte aligned                  */
    FA2_ERR_NO_DEVICE = 4,   /* no usable gfx950 device / HIP runtime failure  */
    FA2_ERR_LAUNCH = 5,      /* the kernel launch failed                       */
    FA2_ERR_SCRATCH_LIMIT = 6 /* fa2_fwd_splitkv_noalloc: the call needs more
                                scratch than FA2_NOALLOC_SCRATCH_BYTES         */
} fa2_status;

/*
 * fa2_fwd -- attention forward pass, asynchronous on `stream`.
 *
 *   q, k, v : device pointers, fp16 (IEEE binary16), shape [B, H, N, d],
 *             contiguous row-major (d fastest).  Read only.
 *   o       : device pointer, fp16 [B, H, N, d], contiguous.  Written: every
 *             element, O rounded once to fp16 (round to nearest even).
 *   lse     : device pointer, fp32 [B, H, N].  Written: natural-log
 *             log-sum-exp of the scaled scores of each query row over its
 *             visible keys.
 *   B, H, N : batch, heads, sequence length (queries = keys = N); each >= 1,
 *             N <= 4194304 (2^22), N * d <= 2^29 and B * H * N <= 2^31 - 1.
 *   d       : head dimension: 32, 64, 96, 128 or 256.
 *   scale   : softmax scale (normally 1/sqrt(d)); finite, with
 *             |scale| * log2(e) * 65504^2 * d <= FLT_MAX (|scale| up to about
 *             5.5e28 / d), so that every scaled score of fp16 inputs is a
 *             finite fp32 number; larger or non-finite values are rejected
 *             with FA2_ERR_INVALID_ARG.  0 gives uniform weights over the
 *             visible keys.  Precision: each weight is exp2 of an fp32
 *             argument whose absolute error is about 2^-24 times the
 *             largest |scale * log2(e) * q.k| of the row; results keep their
 *             accuracy while that magnitude stays below about 2^16, and
 *             carry none once it passes 2^26 (a row may then come out as
 *             zeros, infinities or NaN).
 *   causal  : non-zero: query i sees keys j <= i only (top-left aligned).
 *   stream  : a hipStream_t passed as void*; NULL means the null stream.
 *
 * Ownership: the caller allocates and owns all five buffers.  o and lse must
 * not overlap q, k or v, nor each other (any overlap is rejected).  Alignment: all
 * pointers 16-byte aligned.
 *
 * Errors: all argument checks run before the first HIP call, so a bad call
 * returns FA2_ERR_INVALID_ARG / _UNSUPPORTED / _MISALIGNED without touching
 * the device.  A failed launch returns FA2_ERR_LAUNCH (the HIP error code is
 * then available from fa2_last_hip_error).  The call never prints, throws or
 * synchronises; results are ready once the caller synchronises the stream.
 * NaN or Inf inputs are outside the contract and propagate per IEEE rules.
 */
int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
            int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa2_bwd -- gradients of the forward pass, asynchronous on `stream`.
 *
 * For an upstream gradient dO of O, returns the gradients of <dO, O> (the
 * sum of dO * O over all elements) with respect to Q, K and V:
 *
 *     P  = exp(scale * Q K^T - LSE)  (masked entries 0)
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta_i = dO_i . O_i
 *     dQ = scale * dS K,  dK = scale * dS^T Q
 *
 * S and P are recomputed tile by tile from Q, K and the forward's LSE,
 * never stored ("3.6 Attention I -- the memory problem and FlashAttention
 * principles", 3.6.7: the backward recomputes S and P from the O(N) row
 * statistics kept by the forward; the formulas are the chain rule through
 * the row softmax).
 *
 *   q, k, v : device pointers, fp16 [B, H, N, d], the forward's inputs.
 *   o, lse  : device pointers, the forward's outputs for the same q, k, v,
 *             scale and causal (fp16 [B, H, N, d] and fp32 [B, H, N]).
 *   dout    : device pointer, fp16 [B, H, N, d], the upstream gradient dO.
 *   dq, dk, dv : device pointers, fp16 [B, H, N, d].  Written: every
 *             element, rounded once to fp16 (round to nearest even).
 *   delta   : device pointer, fp32 [B, H, N], caller-owned workspace.
 *             Written: delta_i = sum_c dO_ic * O_ic of each query row, which
 *             the second of the two kernels reads.
 *   B, H, N, scale, causal, stream : as for fa2_fwd.
 *   d       : head dimension: 32, 64, 96 or 128.
 *
 * Ownership: the caller allocates and owns all buffers.  dq, dk, dv and delta
 * must not overlap any input (q, k, v, o, lse, dout) nor each other.
 * Alignment: all pointers 16-byte aligned.  Errors as for fa2_fwd; all
 * argument checks run before the first HIP call.
 */
int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float* delta,
            int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa1_fwd -- the same forward pass (same outputs, within the same tolerance)
 * computed in the FlashAttention-1 loop order, as a comparator for fa2_fwd.
 *
 * "Implementing FlashAttention 1 and 2 forward in Triton", sections
 * "parallelisation unit" and "output accumulation": one program per
 * (batch, head); key/value blocks in the outer loop, every query block in the
 * inner one; after each key/value block the normalised output and the row
 * statistics (m, l) are written to global memory in fp32 and read back for
 * the next block; fp16 only at the end.  Here: one workgroup per
 * (batch, head), 128-key blocks, the fp32 state in `ws`.
 *
 *   q, k, v, o, lse, B, H, N, scale, causal, stream : as for fa2_fwd.
 *   d       : 64 only.  N * d <= 2^27.
 *   ws      : device pointer, caller-owned workspace of at least
 *             fa1_workspace_bytes(B, H, N, d) bytes (fp32 O, m and l of
 *             every row); its contents on entry are ignored, on return
 *             undefined.  ws_bytes is its size.
 * Errors as for fa2_fwd; a workspace that is too small, or overlaps q, k,
 * v, o or lse, is FA2_ERR_INVALID_ARG.
 */
int fa1_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
            size_t ws_bytes, int B, int H, int N, int d, float scale, int causal,
            void* stream);

/* Workspace bytes fa1_fwd needs: B * H * N * (d + 2) * 4 (0 for bad sizes,
 * including B * H * N > 2^31 - 1). */
size_t fa1_workspace_bytes(int B, int H, int N, int d);

/*
 * fa2_fwd_splitkv -- attention of a short query block over a long key/value
 * set (decoding), with the keys split across workgroups; non-causal.
 *
 *     O = softmax(scale * Q K^T) V,  LSE = natural log-sum-exp per query row,
 *
 * for q [B, H, Nq, d] against k, v [B, H, Nk, d].  The keys are split into
 * ranges; each range leaves a partial result normalised over its keys with
 * its own LSE, and the parts are merged with
 * LSE = M + ln sum_s exp(LSE_s - M), O = sum_s exp(LSE_s - LSE) O_s -- the
 * online-softmax recurrence over whole parts ("3.6 Attention I -- the
 * memory problem and FlashAttention principles", 3.6.4; 3.6.9 and 3.6.10
 * name split-key decoding without its steps).
 *
 *   q       : device pointer, fp16 [B, H, Nq, d]; k, v : fp16 [B, H, Nk, d].
 *   o, lse  : device pointers, fp16 [B, H, Nq, d] and fp32 [B, H, Nq].
 *   ws      : device pointer, caller-owned workspace of at least
 *             fa2_splitkv_workspace_bytes(B, H, Nq, Nk, d, n_splits) bytes
 *             (fp32 partial outputs and LSEs); may be NULL when that is 0
 *             (a single range).  ws_bytes is its size.
 *   Nq, Nk  : >= 1, each <= 2^22, N * d <= 2^29 for both.
 *   d       : 32, 64, 96 or 128.
 *   n_splits: requested number of key ranges, 1 .. 4096, or 0 to let the
 *             library choose for the shape; fa2_splitkv_splits returns the
 *             count actually used (never an empty range).
 *   scale, stream : as for fa2_fwd.
 * Errors as for fa2_fwd; a missing or too small workspace, or any overlap of
 * o, lse, ws with an input or each other, is FA2_ERR_INVALID_ARG.
 */
int fa2_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                    void* ws, size_t ws_bytes, int B, int H, int Nq, int Nk, int d,
                    float scale, int n_splits, void* stream);

/* Key ranges fa2_fwd_splitkv uses for these sizes (0 for invalid sizes). */
int fa2_splitkv_splits(int B, int H, int Nq, int Nk, int d, int n_splits);

/* Workspace bytes fa2_fwd_splitkv needs: splits * B * H * Nq * (d + 1) * 4
 * when it uses more than one range, else 0 (also 0 for invalid sizes). */
size_t fa2_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int n_splits);

/* Bytes of the fixed device scratch of fa2_fwd_splitkv_noalloc (8 MiB). */
#define FA2_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * fa2_fwd_splitkv_noalloc -- fa2_fwd_splitkv without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments, kernels and results as fa2_fwd_splitkv (bit
 * for bit, for the same sizes and n_splits), except that the partial outputs
 * and log-sum-exps of the key ranges go to a fixed scratch buffer inside the
 * library: FA2_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from the
 * library's first call on that GPU until the process ends.  The call itself
 * allocates and frees nothing (no hipMalloc, hipFree or allocating library
 * routine); the first call on a device looks the buffer's address up once.
 *
 * Errors as for fa2_fwd_splitkv; a call whose fa2_splitkv_workspace_bytes
 * exceeds FA2_NOALLOC_SCRATCH_BYTES returns FA2_ERR_SCRATCH_LIMIT before any
 * HIP call.  Every call on one GPU shares that GPU's buffer, which keeps the
 * last call's contents: calls that overlap in time on one GPU (several
 * streams, or several host threads) race on it and must be serialised by the
 * caller.  Nothing in the buffer needs to start at zero: each call writes
 * every element it reads.
 */
int fa2_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, int n_splits,
                            void* stream);

/*
 * fa2_lse_merge -- merge n_parts partial attention results over disjoint key
 * sets (the second step of fa2_fwd_splitkv, and the merge of attention
 * computed on key shards elsewhere, e.g. one shard per GPU).
 *
 *   o_parts   : device pointer, fp32 [n_parts, rows, d]: each part's output,
 *               normalised over its own keys.
 *   lse_parts : device pointer, fp32 [n_parts, rows]: each part's natural
 *               log-sum-exp; -inf marks an empty part (its o_parts ignored).
 *   o, lse    : device pointers, fp16 [rows, d] and fp32 [rows]: the merged
 *               result, LSE = M + ln sum_s exp(LSE_s - M), O = sum_s
 *               exp(LSE_s - LSE) O_s (rows whose parts are all empty: O = 0,
 *               LSE = -inf).
 *   n_parts, rows >= 1, n_parts * rows <= 2^31 - 1; d : 32, 64, 96 or 128.
 * Errors as for fa2_fwd; o or lse overlapping an input or each other is
 * FA2_ERR_INVALID_ARG.
 */
int fa2_lse_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                  int n_parts, int rows, int d, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa2_status_string(int status);

/* hipError_t of this thread's last FA2_ERR_LAUNCH / FA2_ERR_NO_DEVICE (0 if none). */
int fa2_last_hip_error(void);

/* Static version string of the library. */
const char* fa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H_ */
