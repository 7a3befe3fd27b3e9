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
 * The same call gives the same bits every time.  The bits of one head do not depend on
 * the other heads or batches of the call, except across the small-grid rule: grids of at
 * most 256 blocks of 128 rows (512 when causal; at d = 64 blocks of 64 rows, 512 or, causal,
 * 1024) give each 32 queries two waves that take alternate 32-key units and add their
 * halves at the end, which rounds differently from one wave per 32 queries (both within
 * the tolerances of the exact result).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 fa_dtype dtype, int causal, float softmax_scale,
                 struct ihipStream_t* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: two fp32 terms per query
 * row, LSE_i * log2(e) and -D_i with D_i = sum_k dO_ik O_ik, rows padded to a multiple
 * of 32 per head, i.e. R = 8 * B * Hq * 32 * ceil(N / 32) bytes.  When the sizes give
 * fewer 128-key blocks (B * Hkv * ceil(N / 128)) than 256 (512 when causal), the dK/dV
 * pass splits each block's query steps into k chunks (k <= 16, at least 32 steps of
 * 32 queries in the longest block's chunks) and the workspace also holds their
 * fp32 partial dK, dV: R rounded up to 256, plus blocks * k * 2 * 128 * d * 4 bytes
 * (at most 512 slots, 64 MiB at d = 128).  Returns 0 for invalid sizes.
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

/*
 * Split-KV forward for decoding: Nq new queries against a long key/value sequence.
 *
 * Follows "Flash Attention" (wiki), sections "Training and autoregressive decoding"
 * and "Flash-Decoding": the key/value sequence is cut into splits, each split is
 * attended with the tiled online-softmax recurrence of fa_fwd, and the partial
 * outputs are merged with their log-sum-exp statistics (fa_lse_combine's rule).
 * The result equals exact attention of the queries over all keys (up to rounding).
 *
 *   q   [B,Hq,Nq,d], k/v [B,Hkv,Nk,d]   inputs, `dtype`, 16-byte aligned
 *   o   [B,Hq,Nq,d]                     output, `dtype` (RNE)
 *   lse [B,Hq,Nq] float32               output: ln sum_j exp(S_ij) (natural log)
 *   The queries are the last Nq positions of the sequence: query i is at position
 *   Nk - Nq + i; with `causal` set it sees keys j <= Nk - Nq + i (requires Nq <= Nk).
 *   num_splits: key splits per (batch, K/V head, 32-row group); 0 picks a default
 *   (fa_fwd_splitkv_num_splits).  The split size is rounded to 32 keys.
 *   workspace, workspace_bytes >= fa_fwd_splitkv_workspace_size(... same num_splits),
 *   16-byte aligned; contents on entry are ignored.
 *   B = 0 or Nq = 0: nothing to do, FA_OK.  Nk = 0 with Nq > 0 is invalid (no keys).
 * Same dtype/d rules and status codes as fa_fwd.
 *
 * As many queries as keys (Nq == Nk >= 128): the same split applied to a whole
 * sequence, for calls whose fa_fwd grid would leave compute units idle (one short
 * sequence, few heads).  Every query block of fa_fwd's forward is computed by
 * num_splits workgroups, each over a contiguous range of 64-key tiles, and the parts are
 * merged by the same log-sum-exp combine; num_splits then counts splits per query block
 * and the split size is rounded to 64 keys.  Default: one split (fa_fwd itself), whose
 * small grids already split each block's keys between two waves of a workgroup.
 */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                         fa_dtype dtype, int causal, float softmax_scale, int64_t num_splits,
                         struct ihipStream_t* stream);

/*
 * Bytes of workspace fa_fwd_splitkv needs: per output row and group of four splits
 * (the splits padded to a multiple of 4), the fp32 partial O (d floats) and partial
 * LSE; with Nq == Nk >= 128, per output row and split.  0 for invalid sizes.
 */
size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                                     fa_dtype dtype, int64_t num_splits);

/* The number of key splits fa_fwd_splitkv uses for num_splits = 0 (before padding to
 * a multiple of 4; with Nq == Nk >= 128, splits per query block); 0 for invalid sizes. */
int64_t fa_fwd_splitkv_num_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d);

/*
 * Merge partial attention results over disjoint key sets ("Flash Attention" wiki,
 * section "Flash-Decoding": partial outputs combined by their log-sum-exp
 * statistics; also the merge step of ring attention).  For each row:
 *   M = max_s LSE_s,  w_s = exp(LSE_s - M),
 *   O = sum_s w_s O_s / sum_s w_s,  LSE = M + ln sum_s w_s,
 * parts with LSE_s = -inf carry no weight; a row whose parts are all -inf gets O = 0
 * and LSE = -inf.
 *
 *   o_parts   [rows, num_parts, d] float32   each O_s normalised over its own keys
 *   lse_parts [rows, num_parts]    float32   natural log
 *   o [rows, d] `dtype` (RNE), lse [rows] float32   outputs
 *   rows >= 0 (0: nothing to do), num_parts >= 1, d in {64, 128}; pointers 16-byte aligned.
 */
fa_status fa_lse_combine(const float* o_parts, const float* lse_parts, void* o, float* lse,
                         int64_t rows, int64_t num_parts, int64_t d, fa_dtype dtype,
                         struct ihipStream_t* stream);

/*
 * Forward pass under the mask family: variable-length (packed) batches, queries and
 * keys of different lengths, sliding windows and block-sparse tile lists.
 *
 * "FlashAttention Primer" sections "FlashAttention-2: better work partitioning"
 * (variable-length entry points, sliding-window attention) and "Hardware, dtype,
 * determinism, and padding caveats" (cu_seqlens); "Flash Attention" (wiki) sections
 * "Block-sparse FlashAttention" (masked blocks skipped, exact on the kept blocks) and
 * "Specialized kernels have boundaries" (causal conventions for unequal lengths).
 *
 * Layout.  Fixed lengths (cu_seqlens_q == cu_seqlens_k == NULL): q, o [B,Hq,Nq,d],
 * k, v [B,Hkv,Nk,d], lse [B,Hq,Nq].  Packed: q, o [Hq,Nq,d] and k, v [Hkv,Nk,d] with
 * Nq, Nk the total rows, lse [Hq,Nq]; sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows likewise (int32, B+1 entries each,
 * device memory, nondecreasing); max_seqlen_q / max_seqlen_k bound the sequence lengths
 * (rows past them are not computed; offsets are clamped to the tensors, so inconsistent
 * arrays give unspecified rows, not invalid accesses).  In fixed mode the max lengths
 * are ignored.
 * Masking.  Within a sequence of Lq queries and Lk keys, query i sits at key position
 * p = i + Lk - Lq (bottom-right alignment).  Key j is visible iff
 * (window_left < 0 or j >= p - window_left) and (window_right < 0 or j <= p + window_right);
 * (-1, -1) is full attention and (-1, 0) causal.  With block lists, queries are cut into
 * blocks of 256 and keys into tiles of 64; block_cnt [B, block_heads, ceil(maxq/256)] and
 * block_idx [B, block_heads, ceil(maxq/256), ceil(maxk/64)] (int32, device; maxq, maxk =
 * Nq, Nk in fixed mode) list, per (sequence, head or all heads, query block), the key
 * tiles to visit in ascending order; other tiles are skipped (their scores masked).
 * block_heads is 1 (one list for all heads) or Hq.  A query that sees no key gets O = 0
 * and LSE = -inf.  softmax_scale, dtype and head sizes as in fa_fwd.  Deterministic;
 * nothing is allocated.
 */
fa_status fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int64_t max_seqlen_q, int64_t max_seqlen_k,
                        int64_t window_left, int64_t window_right, const int32_t* block_cnt,
                        const int32_t* block_idx, int64_t block_heads, float softmax_scale,
                        struct ihipStream_t* stream);

/*
 * Backward pass under the mask family: the gradients of the output of fa_fwd_masked
 * with the same lengths, layout, window and block lists.  "FlashAttention Primer",
 * section "Backward pass: recomputation instead of storage" (P recomputed from the saved
 * LSE), with the masking of fa_fwd_masked; "Flash Attention" (wiki), section
 * "Block-sparse FlashAttention" (tiles off the lists are skipped in both passes).
 *
 *   q, k, v, o, lse, dout   as given to / returned by fa_fwd_masked (o, dout, dq like q;
 *                           dk, dv like k); a row with LSE = -inf contributes nothing
 *   dq, dk, dv              outputs, `dtype`; keys no query sees get dK = dV = 0; rows
 *                           outside every sequence (packed gaps) are not written
 *   block_cnt, block_idx,   as in fa_fwd_masked (NULL, NULL: no lists)
 *   block_heads
 *   workspace               >= fa_bwd_masked_workspace_size(B, Hq, Hkv, max query length,
 *                           max key length, lists given) bytes, 16-byte aligned: row
 *                           terms per (sequence, head) and, with lists, their transpose
 *                           per 128-key block (Hq/Hkv * ceil(maxq/256) below 2^29, else
 *                           FA_ERR_UNSUPPORTED) and 64 MiB of fp32 partial dK/dV for key
 *                           blocks whose lists name many query blocks (split over several
 *                           workgroups, summed in a fixed order)
 * fa_bwd_masked_workspace_size returns 0 for negative sizes or Hq not a multiple of Hkv.
 * Deterministic (no atomics); nothing is allocated.  Errors as in fa_fwd_masked.
 */
size_t fa_bwd_masked_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seqlen_q, int64_t max_seqlen_k,
                                    int block_lists);

fa_status fa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t max_seqlen_q,
                        int64_t max_seqlen_k, int64_t window_left, int64_t window_right, const int32_t* block_cnt,
                        const int32_t* block_idx, int64_t block_heads, float softmax_scale,
                        struct ihipStream_t* stream);

/*
 * FP8 (e4m3) forward pass with per-block scales and incoherent processing.
 *
 * "Flash Attention" (wiki), section "FlashAttention-3": block quantization plus a
 * transform of random signs and a Hadamard matrix applied to queries and keys (the
 * same orthogonal transform on both leaves Q K^T unchanged in exact arithmetic and
 * spreads outliers over all coordinates); "FlashAttention" (explainer), section
 * "What Hopper bought FlashAttention-3": accuracy kept by per-block scaling.  Two steps: quantise Q and K
 * (with the transform) and V once, then run the forward pass on the codes.
 *
 * Quantisation.  x [B,H,N,d] of `dtype` (16-byte aligned); signs: d floats of +1/-1
 * on the device, or NULL for no transform.  With signs, each row becomes
 * x diag(signs) H_d / sqrt(d) (H_d the Sylvester Hadamard matrix), formed exactly in
 * fp64 with one fp64 multiplication by the fp64 value nearest 1/sqrt(d), then rounded
 * to fp32.  Every block of block_rows consecutive rows of a head (64, 128 or 256; the
 * last block may be short) gets the power-of-two scale 2^e, e the smallest integer
 * with max|value| <= 448 * 2^e (e = 0 for an all-zero block), and the codes are
 * e4m3(value / 2^e), rounded to nearest even.  Non-finite inputs, or values past the
 * fp32 range after the transform, give unspecified codes.
 *   fa_fp8_quantize_rows: codes [B,H,N,d] bytes (16-byte aligned), scales float
 *       [B,H,ceil(N/block_rows)] (4-byte aligned).  For queries and keys.
 *   fa_fp8_quantize_v:    codes in the value-tile layout [B,H,ceil(N/64),d,64] bytes
 *       (fa_fp8_v_codes_bytes): per 64-key tile the transposed [d][64] block, keys
 *       permuted so that position 32h + 16t + 4a + b holds key 32t + 8a + 4h + b;
 *       keys past N are code 0.  Scales as above.  No transform.
 *
 * fa_fwd_fp8.  q8 [B,Hq,N,d] and k8 [B,Hkv,N,d] row codes, v8 value tiles of
 * [B,Hkv,N,d], their scales with block sizes block_q and block_kv (64, 128 or 256;
 * scales must be powers of two, as the quantisers write them); o [B,Hq,N,d] bf16,
 * lse [B,Hq,N] float32 (natural log).  S = softmax_scale * Q' K'^T over the
 * dequantised codes (scale * value); P is rounded to e4m3 for the product with V
 * (P <= 256 by the rescaling threshold); the row sums behind O's normalisation and
 * the LSE use the unrounded fp32 P.  Grouping and causal masking as in fa_fwd.
 * Outputs are deterministic.  Buffers are the caller's; nothing is allocated.
 */
size_t fa_fp8_v_codes_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

fa_status fa_fp8_quantize_rows(const void* x, const float* signs, void* codes, float* scales, int64_t B,
                               int64_t H, int64_t N, int64_t d, fa_dtype dtype, int64_t block_rows,
                               struct ihipStream_t* stream);

fa_status fa_fp8_quantize_v(const void* x, void* codes, float* scales, int64_t B, int64_t H, int64_t N, int64_t d,
                            fa_dtype dtype, int64_t block_rows, struct ihipStream_t* stream);

fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scales, const float* k_scales,
                     const float* v_scales, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                     int64_t d, int64_t block_q, int64_t block_kv, int causal, float softmax_scale,
                     struct ihipStream_t* stream);

/*
 * Backward pass without a caller workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and bits as fa_bwd minus the workspace: the
 * workspace fa_bwd_workspace_size() reports for these sizes lives in a static device
 * array of 64 MiB (67108864 bytes) per GPU, created when the
 * library's code is loaded on that GPU and held until the process ends.  Nothing is
 * allocated or freed by the call.  Sizes whose workspace exceeds that maximum return
 * FA_ERR_INVALID_ARGUMENT (use fa_bwd).  All calls on one GPU share its array, so calls
 * that may overlap in time on one GPU (different streams, different threads without
 * ordering) race and give undefined results; calls in one stream are ordered and safe.
 * The first call on each device, with that device current, looks up the array's address
 * (hipGetSymbolAddress); a failure there returns FA_ERR_HIP.
 */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t N, int64_t d, fa_dtype dtype, int causal, float softmax_scale,
                         struct ihipStream_t* stream);

/*
 * Error reporting.  The "Flash Attention" wiki (sections "Framework integration" and
 * "Specialized kernels have boundaries") describes fused kernels that reject inputs
 * outside their specialisation, and a forced backend that turns an unsupported call into
 * an error instead of quietly running another kernel.  This library does the same: a
 * call it cannot serve returns a status and runs nothing; there is no fallback.  These
 * two functions let the caller report why.
 *
 * fa_status_string: static, human-readable name of a status code ("FA_ERR_UNKNOWN" for
 * a value outside the enum).  The string is owned by the library and never freed.
 *
 * fa_last_error: detail text of the failure of the most recent call on the calling thread.
 * Every entry point that returns an fa_status clears it on entry, so it is "" after a
 * successful call.  The buffer is thread-local and owned by the library: the pointer
 * stays valid for the thread's life, and the next such call on that thread rewrites it.
 */
const char* fa_status_string(fa_status s);

const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
