/*
 * fa.h — C ABI of the fused exact-attention library for MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention,
 *     S = softmax_scale * Q K^T,  P = row-softmax(S),  O = P V,
 * as defined in "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4"
 * (section "Why attention is quadratic"), with the tiled online-softmax forward
 * of the same page (section "FlashAttention-1: tiling plus online softmax",
 * Figures 3 and 4) and the recomputing backward (section "Backward pass:
 * recomputation instead of storage", Figure 5).
 *
 * Layout.  Every tensor is dense, contiguous, row-major:
 *     q, o, dout, dq : [B, Hq,  N, d]   elements of `dtype`
 *     k, v, dk, dv   : [B, Hkv, N, d]   elements of `dtype`
 *     lse            : [B, Hq,  N]      float32
 * Query head hq uses key/value head hq / (Hq / Hkv) (contiguous groups; Hkv == Hq
 * is multi-head, Hkv == 1 multi-query attention).  Query and key lengths are
 * equal (N).  With `causal` set, query i attends to keys j <= i.
 *
 * Ownership and execution.  The caller owns every buffer; pointers are device
 * pointers (HIP device memory of the current device).  Nothing is allocated by
 * fa_fwd; fa_bwd uses only the caller's workspace.  All work is enqueued on
 * `stream` (NULL = the default stream); calls return without synchronising, and
 * the inputs must stay alive and unmodified until the stream passes the call.
 *
 * Errors.  Arguments are validated on the host before any HIP call; an invalid
 * call returns a status and enqueues nothing.  Outputs are undefined after a
 * failed call.  No exception or abort crosses this interface.  fa_last_error()
 * returns a thread-local description of the last failure on the calling thread.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t *` */

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad sizes, bad scale, small workspace */
  FA_ERR_UNSUPPORTED = 2,      /* head dimension other than 64 or 128, unknown dtype */
  FA_ERR_HIP = 3               /* a HIP runtime call or kernel launch failed */
} fa_status;

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/*
 * Forward pass: O and the per-row log-sum-exp.
 *
 * Follows the tiled forward of "FlashAttention Primer" (section "FlashAttention-1:
 * tiling plus online softmax", Figure 4) with the work split of its section
 * "FlashAttention-2: better work partitioning" (Figure 6: one workgroup per
 * (batch, head, query block), no atomics, bitwise deterministic).
 *
 *   q [B,Hq,N,d], k/v [B,Hkv,N,d]  inputs, `dtype` elements, 16-byte aligned
 *   o   [B,Hq,N,d]                  output, `dtype` (round-to-nearest-even)
 *   lse [B,Hq,N] float32            output: ln sum_j exp(S_ij) over the masked,
 *                                   scaled scores of row i (natural log)
 *   B >= 0, N >= 0 (either 0: nothing to do, FA_OK); Hq >= 1, Hkv >= 1, Hq % Hkv == 0;
 *   d in {64, 128}; softmax_scale finite and > 0 (callers normally pass 1/sqrt(d)).
 * Returns FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 fa_dtype dtype, int causal, float softmax_scale,
                 struct ihipStream_t* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: two fp32 terms per query
 * row, LSE_i * log2(e) and -D_i with D_i = sum_k dO_ik O_ik, rows padded to a multiple
 * of 32 per head, i.e. 8 * B * Hq * 32 * ceil(N / 32) bytes.  Returns 0 for invalid
 * sizes.
 */
size_t fa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                             fa_dtype dtype, int causal);

/*
 * Backward pass by recomputation: dQ, dK, dV from Q, K, V, O, the saved LSE and dO.
 *
 * Follows "FlashAttention Primer" (section "Backward pass: recomputation instead of
 * storage", Figure 5): P is recomputed block by block from the saved LSE.  The
 * gradient is the full softmax-attention gradient, dS = P * (dP - D) with
 * D_i = sum_k dO_ik O_ik, and dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO
 * (dK, dV summed over the query heads sharing a K/V head).  dQ and dK/dV come
 * from two passes that each own their output, with no atomic adds, so the
 * result is bitwise reproducible run to run (the deterministic option discussed
 * in the Primer's same section).
 *
 *   q, k, v, o, lse, dout : as produced for / by fa_fwd with the same arguments
 *   dq [B,Hq,N,d], dk/dv [B,Hkv,N,d]   outputs, `dtype`
 *   workspace, workspace_bytes          >= fa_bwd_workspace_size(...), 16-byte aligned;
 *                                       contents on entry are ignored
 * Same size rules and status codes as fa_fwd.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 fa_dtype dtype, int causal, float softmax_scale,
                 struct ihipStream_t* stream);

/* Static, human-readable name of a status code. */
const char* fa_status_string(fa_status s);

/* Thread-local detail text of the last failed call on this thread ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
