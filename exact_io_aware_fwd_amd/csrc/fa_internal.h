// Launch-side interface between the C ABI (fa_api.cpp) and the kernels.
// Arguments reaching these functions have been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N;
  float scale;        // softmax scale
  float scale_log2;   // softmax scale * log2(e)
  // Mask family (the general kernel only).  Fixed lengths: q [B,Hq,N,d], k/v [B,Hkv,Nk,d].
  // Packed (cu_q != null): q [Hq,N,d], k/v [Hkv,Nk,d], sequence b = rows cu[b] .. cu[b+1]-1.
  int Nk = 0;
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int maxq = 0, maxk = 0;     // longest sequence (grid size; rows past it are not computed)
  int wl = -1, wr = -1;       // window (left, right), -1 = unbounded
  const int* bcnt = nullptr;  // block lists: counts [B, bheads, bnq]
  const int* bidx = nullptr;  //              tiles  [B, bheads, bnq, bcap], ascending
  int bheads = 1, bnq = 0, bcap = 0;
  // Key split (the general kernel, fixed lengths, no block lists): workgroup split s of
  // ksplit sees only keys [s*kchunk, (s+1)*kchunk) and writes its part of every row,
  // O / l in fp32 to opart [rows, ksplit, d] and its LSE to lpart [rows, ksplit]
  // (rows in [B, Hq, N] order), to be merged by the LSE combine.
  int ksplit = 1, kchunk = 0;
  float* opart = nullptr;
  float* lpart = nullptr;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* rowterm;  // workspace: per (b, hq) and 32-row block, 32 x LSE_i * log2 e then 32 x -D_i (fp32)
  int B, Hq, Hkv, N;
  float scale;
  float scale_log2;
  // Mask family (the general kernels only), as in FwdArgs; the row terms are padded per
  // (batch, head) to ceil(maxq / 32) blocks.
  int Nk = 0;
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int maxq = 0, maxk = 0;
  int wl = -1, wr = -1;
  // Block lists as in FwdArgs, and (workspace, after the row terms) their transpose for
  // the dK/dV pass: per (batch, K/V head, 128-key block) a record of rstride ints; the
  // chunk plan (per record: chunks, first slot); the slot table; the partial dK/dV slots.
  const int* bcnt = nullptr;
  const int* bidx = nullptr;
  int bheads = 1, bnq = 0, bcap = 0;
  int* runs = nullptr;
  long long rstride = 0;
  int* plan = nullptr;
  int* table = nullptr;
  float* pool = nullptr;
  // fa_bwd with few key blocks for the CUs: the query steps of every key block are split
  // into ksplit chunks, whose partial dK, dV go to `pool` (ksplit consecutive slots per
  // key block, record = (batch * Hkv + K/V head) * key blocks + key block)
  int ksplit = 1;
  int kblock = 128;   // fa_bwd: keys per dK/dV record, 256 (64 keys a wave) or 128 (32)
  int rowterm_here = 0;   // fa_bwd: the dQ pass forms the row terms and writes them
};

// Split-KV forward (decoding): queries [B, Hq, Nq, d] against keys/values [B, Hkv, Nk, d].
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* opart;    // workspace: partial O per (row, 4-split workgroup), [B*Hq*Nq, S4/4, d] fp32
  float* lpart;    // workspace: partial LSE per (row, workgroup), [B*Hq*Nq, S4/4] fp32 (natural log)
  int B, Hq, Hkv, Nq, Nk;
  int RG;          // 32-row groups per (batch, K/V head): ceil(Hq/Hkv * Nq / 32)
  int C;           // keys per split (a multiple of 32)
  int S4;          // splits, padded to a multiple of 4 (one wave each)
  float scale;
  float scale_log2;
};

// How the keys are split.  num_splits = 0 picks a count that gives about four waves
// per CU in one round (1024 waves on 256 CUs).
struct SplitPlan {
  int RG, C, S4;
};
inline SplitPlan plan_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t num_splits) {
  SplitPlan p;
  const int64_t G = Hq / Hkv;
  p.RG = (int)((G * Nq + 31) / 32);
  const int64_t units = (Nk + 31) / 32;
  int64_t S = num_splits;
  if (S <= 0) {
    const int64_t groups = B * Hkv * p.RG;
    S = (1024 + groups - 1) / groups;
  }
  if (S > units) S = units;
  if (S < 1) S = 1;
  const int64_t per = (units + S - 1) / S;             // units per split
  p.C = (int)(per * 32);
  const int64_t used = (Nk + p.C - 1) / p.C;           // non-empty splits
  p.S4 = (int)((used + 3) / 4 * 4);
  return p;
}
// Split-KV with as many queries as keys (a prefill whose own grid leaves CUs idle): the
// general forward kernel with a key split, then the LSE combine.  Default: one split, which
// is fa_fwd itself, writing O and LSE directly (its small grids split each block's keys
// between two waves without fp32 partials, faster than two or more key splits: 16 heads of
// 1024 causal, d = 128: 0.0225 ms against 0.0276 with two; d = 64: 0.0129 against 0.0199).
constexpr int64_t kPrefillSplitMinRows = 128;   // Nq == Nk at least this long takes this route
struct PrefillSplit {
  int S, C;   // splits used, keys per split (a multiple of 64)
};
inline bool splitkv_is_prefill(int64_t Nq, int64_t Nk) { return Nq == Nk && Nq >= kPrefillSplitMinRows; }
inline PrefillSplit plan_prefill_split(int64_t N, int64_t num_splits) {
  const int64_t tiles = (N + 63) / 64;
  int64_t S = num_splits;
  if (S <= 0) S = 1;
  if (S > tiles) S = tiles;
  if (S < 1) S = 1;
  const int64_t per = (tiles + S - 1) / S;
  PrefillSplit p;
  p.C = (int)(per * 64);
  p.S = (int)((tiles + per - 1) / per);
  return p;
}
inline size_t prefill_opart_bytes(int64_t B, int64_t Hq, int64_t N, int64_t d, const PrefillSplit& p) {
  return p.S == 1 ? 0 : (size_t)((B * Hq * N * p.S * d * 4 + 255) / 256 * 256);
}
inline size_t prefill_workspace_bytes(int64_t B, int64_t Hq, int64_t N, int64_t d, const PrefillSplit& p) {
  return p.S == 1 ? 0 : prefill_opart_bytes(B, Hq, N, d, p) + (size_t)((B * Hq * N * p.S * 4 + 255) / 256 * 256);
}
inline size_t splitkv_opart_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t d, const SplitPlan& p) {
  return (size_t)((B * Hq * Nq * (p.S4 / 4) * d * 4 + 255) / 256 * 256);
}
inline size_t splitkv_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t d, const SplitPlan& p) {
  return splitkv_opart_bytes(B, Hq, Nq, d, p) + (size_t)((B * Hq * Nq * (p.S4 / 4) * 4 + 255) / 256 * 256);
}

// FP8 block quantisation: one workgroup of block_rows * d / 32 threads per scale block.
struct QuantArgs {
  const void* x;        // [B, H, N, d] fp16/bf16
  const float* signs;   // [d] of +-1 (transform) or null
  uint8_t* codes;       // rows: [B, H, N, d]; value tiles: [B, H, ceil(N/64), d, 64]
  float* scales;        // [B, H, nblk] powers of two
  int BH, N, block_rows, nblk;
  double inv_sqrt_d;    // the fp64 value nearest 1/sqrt(d)
};

// FP8 forward: codes and power-of-two block scales of the transformed Q and K and of V
// (value tiles as written by the quantiser), bf16 output.
struct Fp8FwdArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* qs;
  const float* ks;
  const float* vs;
  void* o;
  float* lse;
  int B, Hq, Hkv, N;
  int qshift, kvshift;  // log2 of the query and key/value block rows
  float scale_log2;     // softmax scale * log2(e)
};

// Return a hipError_t from the launches (hipSuccess when all were enqueued).
hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16, bool causal, hipStream_t stream);
hipError_t launch_fwd_masked(const FwdArgs& a, int d, bool bf16, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16, bool causal, hipStream_t stream);
hipError_t launch_bwd_masked(const BwdArgs& a, int d, bool bf16, hipStream_t stream);
hipError_t launch_splitkv(const DecodeArgs& a, int d, bool bf16, bool causal, hipStream_t stream);
// mode 0: rows with the transform, 1: rows, 2: value tiles
hipError_t launch_fp8_quant(const QuantArgs& a, int d, bool bf16, int mode, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_lse_combine(const float* opart, const float* lpart, void* o, float* lse, long long rows, int S,
                              int d, bool bf16, hipStream_t stream);

// Workspace of the backward pass: two fp32 row terms per query row, rows padded to a
// multiple of 32 per head (256 bytes per 32-row block).
inline size_t bwd_rowterm_bytes(int64_t B, int64_t Hq, int64_t N) {
  return (size_t)(B * Hq * ((N + 31) / 32) * 256);
}
// fa_bwd's dK/dV pass: records of 256 keys (64 keys a wave) or 128 (32 a wave).  A
// record's query steps may be split into k chunks (at most 16) whose fp32 partial dK, dV
// are summed in chunk order afterwards, so that the records and their chunks give the
// CUs 256 workgroups, or 512 when causal (where the records' step counts range over the
// whole sequence).  The longest record's chunks keep at least kBwdSplitMinSteps steps
// (256-key records: kBwdSplitMinSteps256, their partials being twice as large), below
// which writing and summing the partials cost more than the balance gains.  256-key
// records are used whenever they give as many workgroups as 128-key ones (half the LDS
// reads per product); 128-key ones remain for the smaller grids.
constexpr int kBwdSplitMinSteps = 32;
constexpr int kBwdSplitMinSteps256 = 256;
struct BwdDensePlan {
  int kblock;   // keys per record
  int ksplit;   // chunks per record (1: no split)
};
inline int bwd_dense_chunks(int64_t records, int64_t steps, bool causal, int min_steps) {
  if (records <= 0) return 1;
  int64_t k = (causal ? 512 : 256) / records;
  k = k < 16 ? k : 16;
  k = k < steps / min_steps ? k : steps / min_steps;
  return (int)(k > 1 ? k : 1);
}
inline BwdDensePlan bwd_dense_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, bool causal) {
  if (Hkv <= 0 || N <= 0) return {128, 1};
  const int64_t steps = (Hq / Hkv) * ((N + 31) / 32);   // the longest record's steps
  const int64_t r256 = B * Hkv * ((N + 255) / 256), r128 = B * Hkv * ((N + 127) / 128);
  const int k256 = bwd_dense_chunks(r256, steps, causal, kBwdSplitMinSteps256);
  const int k128 = bwd_dense_chunks(r128, steps, causal, kBwdSplitMinSteps);
  if (r256 >= (causal ? 512 : 256) || r256 * k256 >= r128 * k128) return {256, k256};
  return {128, k128};
}
// fa_bwd workspace: the row terms, then (split) the partial slots, 2 x kblock keys x d
// fp32 each, from a 256-byte boundary.
inline size_t bwd_pool_offset(int64_t B, int64_t Hq, int64_t N) {
  return (bwd_rowterm_bytes(B, Hq, N) + 255) / 256 * 256;
}
inline size_t bwd_dense_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, bool causal) {
  const BwdDensePlan pl = bwd_dense_plan(B, Hq, Hkv, N, causal);
  if (pl.ksplit == 1) return bwd_rowterm_bytes(B, Hq, N);
  const int64_t records = B * Hkv * ((N + pl.kblock - 1) / pl.kblock);
  return bwd_pool_offset(B, Hq, N) + (size_t)records * pl.ksplit * 2 * pl.kblock * (size_t)d * 4;
}
// Block lists in the masked backward.  The dK/dV pass splits a key block whose
// transposed list names more query steps than its share (total steps / kBwdTargetChunks,
// at least kBwdMinChunk) into chunks run by separate workgroups; each chunk writes fp32
// partial dK, dV (128 keys x d <= 128, both tensors) into one of kBwdSlots slots, and a
// reduction sums them in chunk order.
constexpr int kBwdSlots = 512;
constexpr int kBwdTargetChunks = 256;
constexpr int kBwdMinChunk = 64;
// per (batch, K/V head, 128-key block): two header ints and three ints per (query head of
// the group, 256-query block)
inline int64_t bwd_runs_stride(int64_t Hq, int64_t Hkv, int64_t maxq) {
  return 2 + 3 * (Hq / Hkv) * ((maxq + 255) / 256);
}
// Byte offsets of the regions of the masked backward's workspace with block lists (the
// row terms come first); `end` is its size.
struct BwdListLayout {
  size_t runs, plan, table, pool, end;
};
inline BwdListLayout bwd_list_layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t maxq, int64_t maxk) {
  auto align = [](int64_t x) { return (size_t)((x + 255) / 256 * 256); };
  const int64_t nrec = B * Hkv * ((maxk + 127) / 128);
  BwdListLayout L;
  L.runs = bwd_rowterm_bytes(B, Hq, maxq);
  L.plan = L.runs + align(nrec * bwd_runs_stride(Hq, Hkv, maxq) * 4);
  L.table = L.plan + align(nrec * 2 * 4);
  L.pool = L.table + align((1 + 2 * (int64_t)kBwdSlots) * 4);
  L.end = L.pool + (size_t)kBwdSlots * 2 * 128 * 128 * 4;
  return L;
}

}  // namespace fa
