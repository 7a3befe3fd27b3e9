// C ABI of the attention library: host-side validation, then launches on the
// caller's stream.  See include/fa.h for the contract of every entry point.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "fa_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

thread_local char g_last_error[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Size checks shared by the forward and backward passes.  Sets *empty when
// there is nothing to compute (B == 0 or N == 0).
fa_status check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, fa_dtype dtype,
                      bool* empty) {
  if (B < 0 || N < 0) return fail(FA_ERR_INVALID_ARGUMENT, "B and N must be >= 0 (B=%lld N=%lld)",
                                  (long long)B, (long long)N);
  if (Hq < 1 || Hkv < 1) return fail(FA_ERR_INVALID_ARGUMENT, "Hq and Hkv must be >= 1 (Hq=%lld Hkv=%lld)",
                                     (long long)Hq, (long long)Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARGUMENT, "Hq (%lld) must be a multiple of Hkv (%lld)",
                                 (long long)Hq, (long long)Hkv);
  if (d < 1) return fail(FA_ERR_INVALID_ARGUMENT, "d must be >= 1 (d=%lld)", (long long)d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %lld not supported (64 or 128)",
                                       (long long)d);
  if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  // Index arithmetic inside the kernels: per-head offsets are 64-bit; rows,
  // heads and block counts are 32-bit.
  if (B > INT_MAX || Hq > INT_MAX || N > INT_MAX / 2 || B * Hq > INT_MAX || N * d > INT_MAX)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes exceed the supported index range");
  const int64_t nqb = (N + 255) / 256;
  if (B * Hq > 0 && nqb > (int64_t)UINT_MAX / (B * Hq))
    return fail(FA_ERR_INVALID_ARGUMENT, "grid size exceeds the launch limit");
  *empty = (B == 0 || N == 0);
  return FA_OK;
}

fa_status check_scale(float s) {
  if (!std::isfinite(s) || !(s > 0.f))
    return fail(FA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0 (got %g)", (double)s);
  return FA_OK;
}

fa_status check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return FA_OK;
}

}  // namespace

namespace {

// Size checks of the split-KV forward.  Sets *empty when there is nothing to compute.
fa_status check_splitkv_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                              fa_dtype dtype, int causal, int64_t num_splits, bool* empty) {
  if (B < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "B, Nq and Nk must be >= 0 (B=%lld Nq=%lld Nk=%lld)", (long long)B,
                (long long)Nq, (long long)Nk);
  if (Hq < 1 || Hkv < 1) return fail(FA_ERR_INVALID_ARGUMENT, "Hq and Hkv must be >= 1 (Hq=%lld Hkv=%lld)",
                                     (long long)Hq, (long long)Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARGUMENT, "Hq (%lld) must be a multiple of Hkv (%lld)",
                                 (long long)Hq, (long long)Hkv);
  if (d < 1) return fail(FA_ERR_INVALID_ARGUMENT, "d must be >= 1 (d=%lld)", (long long)d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %lld not supported (64 or 128)",
                                       (long long)d);
  if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (num_splits < 0) return fail(FA_ERR_INVALID_ARGUMENT, "num_splits must be >= 0 (got %lld)", (long long)num_splits);
  // per-head K/V byte offsets are 32-bit in the kernel; rows and splits are 32-bit
  if (B > INT_MAX || Hq > INT_MAX || Nq > INT_MAX || Nk > INT_MAX / 2 || Nk * d > INT_MAX / 2 ||
      B * Hq > INT_MAX || B * Hq * Nq > INT_MAX || num_splits > INT_MAX)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes exceed the supported index range");
  *empty = (B == 0 || Nq == 0);
  if (*empty) return FA_OK;
  if (Nk == 0) return fail(FA_ERR_INVALID_ARGUMENT, "Nk = 0: the queries have no keys");
  if (causal && Nq > Nk)
    return fail(FA_ERR_INVALID_ARGUMENT, "causal needs Nq <= Nk (Nq=%lld Nk=%lld)", (long long)Nq, (long long)Nk);
  if (fa::splitkv_is_prefill(Nq, Nk)) {
    const fa::PrefillSplit p = fa::plan_prefill_split(Nq, num_splits);
    if (B * Hq * ((Nq + 191) / 192) * p.S > (int64_t)UINT_MAX || Nq * d > INT_MAX)
      return fail(FA_ERR_INVALID_ARGUMENT, "grid size exceeds the launch limit");
    return FA_OK;
  }
  const fa::SplitPlan p = fa::plan_splits(B, Hq, Hkv, Nq, Nk, num_splits);
  if ((int64_t)B * Hkv * p.RG * (p.S4 / 4) > (int64_t)UINT_MAX)
    return fail(FA_ERR_INVALID_ARGUMENT, "grid size exceeds the launch limit");
  return FA_OK;
}

}  // namespace

namespace {

bool fp8_block_ok(int64_t b) { return b == 64 || b == 128 || b == 256; }
int log2_block(int64_t b) { return b == 64 ? 6 : b == 128 ? 7 : 8; }

// The fp64 value nearest 1/sqrt(d) for d a power of two: 2^(-k/2) for even k = log2 d,
// else the fp64 value nearest sqrt(2) times 2^(-(k+1)/2) (scaling by 2^j commutes
// with rounding, and sqrt is correctly rounded).
double inv_sqrt_pow2(int64_t d) {
  int k = 0;
  while ((int64_t(1) << k) < d) ++k;
  return (k % 2 == 0) ? std::ldexp(1.0, -k / 2) : std::ldexp(std::sqrt(2.0), -(k + 1) / 2);
}

fa_status check_ptr4(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", name);
  return FA_OK;
}

// Size checks of the FP8 quantisers.  Sets *empty when there is nothing to do.
fa_status check_fp8_quant(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dtype, int64_t block_rows,
                          bool* empty) {
  if (B < 0 || N < 0) return fail(FA_ERR_INVALID_ARGUMENT, "B and N must be >= 0 (B=%lld N=%lld)", (long long)B,
                                  (long long)N);
  if (H < 1) return fail(FA_ERR_INVALID_ARGUMENT, "H must be >= 1 (H=%lld)", (long long)H);
  if (d < 1) return fail(FA_ERR_INVALID_ARGUMENT, "d must be >= 1 (d=%lld)", (long long)d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %lld not supported (64 or 128)",
                                       (long long)d);
  if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (!fp8_block_ok(block_rows))
    return fail(FA_ERR_INVALID_ARGUMENT, "block_rows must be 64, 128 or 256 (got %lld)", (long long)block_rows);
  if (B > INT_MAX || H > INT_MAX || N > INT_MAX / 2 || B * H > INT_MAX || N * d > INT_MAX)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes exceed the supported index range");
  const int64_t nblk = (N + block_rows - 1) / block_rows;
  if (B * H > 0 && nblk > (int64_t)UINT_MAX / (B * H))
    return fail(FA_ERR_INVALID_ARGUMENT, "grid size exceeds the launch limit");
  *empty = (B == 0 || N == 0);
  return FA_OK;
}

fa_status run_fp8_quant(const void* x, const float* signs, void* codes, float* scales, int64_t B, int64_t H,
                        int64_t N, int64_t d, fa_dtype dtype, int64_t block_rows, int mode, hipStream_t stream) {
  bool empty = false;
  fa_status st = check_fp8_quant(B, H, N, d, dtype, block_rows, &empty);
  if (st != FA_OK || empty) return st;
  if ((st = check_ptr(x, "x")) != FA_OK || (st = check_ptr(codes, "codes")) != FA_OK ||
      (st = check_ptr4(scales, "scales")) != FA_OK)
    return st;
  if (mode == 0 && (st = check_ptr4(signs, "signs")) != FA_OK) return st;
  fa::QuantArgs a;
  a.x = x;
  a.signs = signs;
  a.codes = static_cast<uint8_t*>(codes);
  a.scales = scales;
  a.BH = (int)(B * H);
  a.N = (int)N;
  a.block_rows = (int)block_rows;
  a.nblk = (int)((N + block_rows - 1) / block_rows);
  a.inv_sqrt_d = inv_sqrt_pow2(d);
  const hipError_t err = fa::launch_fp8_quant(a, (int)d, dtype == FA_BF16, mode, stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "quantisation launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

// Validation shared by the mask-family entry points; fills the common fields of args.
template <class Args>
fa_status check_masked(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype,
                       const int32_t* cu_q, const int32_t* cu_k, int64_t max_q, int64_t max_k, int64_t wl,
                       int64_t wr, float scale, bool* empty, Args& a) {
  const bool packed = cu_q != nullptr || cu_k != nullptr;
  if (packed && (cu_q == nullptr || cu_k == nullptr))
    return fail(FA_ERR_INVALID_ARGUMENT, "give both cu_seqlens_q and cu_seqlens_k, or neither");
  if (Nk < 0) return fail(FA_ERR_INVALID_ARGUMENT, "Nk must be >= 0 (Nk=%lld)", (long long)Nk);
  fa_status st = check_sizes(B, Hq, Hkv, std::max(Nq, Nk), d, dtype, empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  const int64_t maxq = packed ? max_q : Nq, maxk = packed ? max_k : Nk;
  if (packed && (max_q < 0 || max_k < 0 || max_q > Nq || max_k > Nk))
    return fail(FA_ERR_INVALID_ARGUMENT, "max_seqlen_q/k must be in [0, Nq] / [0, Nk] (got %lld, %lld)",
                (long long)max_q, (long long)max_k);
  if (wl < -1 || wr < -1 || wl > INT_MAX / 2 || wr > INT_MAX / 2)
    return fail(FA_ERR_INVALID_ARGUMENT, "window sides must be -1 (unbounded) or >= 0 (got %lld, %lld)",
                (long long)wl, (long long)wr);
  if (packed && ((st = check_ptr4(cu_q, "cu_seqlens_q")) != FA_OK || (st = check_ptr4(cu_k, "cu_seqlens_k")) != FA_OK))
    return st;
  *empty = *empty || B == 0 || maxq == 0;
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.N = (int)Nq;
  a.Nk = (int)Nk;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.maxq = (int)maxq;
  a.maxk = (int)maxk;
  a.wl = (int)wl;
  a.wr = (int)wr;
  return FA_OK;
}

// Block lists of the masked entry points (validated after check_masked has filled a):
// both arrays or neither, block_heads 1 or Hq, 4-byte aligned unless there is no work.
template <class Args>
fa_status check_lists(const int32_t* block_cnt, const int32_t* block_idx, int64_t block_heads, int64_t Hq,
                      bool empty, Args& a) {
  if ((block_cnt == nullptr) != (block_idx == nullptr))
    return fail(FA_ERR_INVALID_ARGUMENT, "give both block_cnt and block_idx, or neither");
  if (block_idx != nullptr && block_heads != 1 && block_heads != Hq)
    return fail(FA_ERR_INVALID_ARGUMENT, "block_heads must be 1 or Hq (got %lld)", (long long)block_heads);
  fa_status st = FA_OK;
  if (!empty && block_idx != nullptr && ((st = check_ptr4(block_cnt, "block_cnt")) != FA_OK ||
                                         (st = check_ptr4(block_idx, "block_idx")) != FA_OK))
    return st;
  a.bcnt = block_cnt;
  a.bidx = block_idx;
  a.bheads = block_idx ? (int)block_heads : 1;
  a.bnq = (a.maxq + 255) / 256;
  a.bcap = (a.maxk + 63) / 64;
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error; }

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t N, int64_t d, fa_dtype dtype, int causal, float softmax_scale,
                 struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  bool empty = false;
  fa_status st = check_sizes(B, Hq, Hkv, N, d, dtype, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if ((st = check_ptr(q, "q")) != FA_OK || (st = check_ptr(k, "k")) != FA_OK ||
      (st = check_ptr(v, "v")) != FA_OK || (st = check_ptr(o, "o")) != FA_OK ||
      (st = check_ptr(lse, "lse")) != FA_OK)
    return st;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.N = (int)N;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t err = fa::launch_fwd(a, (int)d, dtype == FA_BF16, causal != 0, (hipStream_t)stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "forward launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

size_t fa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, fa_dtype dtype,
                             int causal) {
  bool empty = false;
  if (check_sizes(B, Hq, Hkv, N, d, dtype, &empty) != FA_OK) return 0;
  return fa::bwd_dense_bytes(B, Hq, Hkv, N, d, causal != 0);
}

namespace {

// fa_bwd after argument checks common to it and fa_bwd_noalloc (the workspace pointer and
// size are checked by the callers).
fa_status bwd_checked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, void* workspace, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t N, int64_t d, fa_dtype dtype, int causal, float softmax_scale,
                      struct ihipStream_t* stream) {
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.rowterm = static_cast<float*>(workspace);
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.N = (int)N;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * kLog2e;
  const fa::BwdDensePlan plan = fa::bwd_dense_plan(B, Hq, Hkv, N, causal != 0);
  a.kblock = plan.kblock;
  a.ksplit = plan.ksplit;
  if (a.ksplit > 1) a.pool = reinterpret_cast<float*>(static_cast<char*>(workspace) + fa::bwd_pool_offset(B, Hq, N));
  const hipError_t err = fa::launch_bwd(a, (int)d, dtype == FA_BF16, causal != 0, (hipStream_t)stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

fa_status bwd_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t N, int64_t d, fa_dtype dtype, float softmax_scale, bool* empty) {
  fa_status st = check_sizes(B, Hq, Hkv, N, d, dtype, empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  if (*empty) return FA_OK;
  if ((st = check_ptr(q, "q")) != FA_OK || (st = check_ptr(k, "k")) != FA_OK ||
      (st = check_ptr(v, "v")) != FA_OK || (st = check_ptr(o, "o")) != FA_OK ||
      (st = check_ptr(lse, "lse")) != FA_OK || (st = check_ptr(dout, "dout")) != FA_OK ||
      (st = check_ptr(dq, "dq")) != FA_OK || (st = check_ptr(dk, "dk")) != FA_OK ||
      (st = check_ptr(dv, "dv")) != FA_OK)
    return st;
  return FA_OK;
}

}  // namespace

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, fa_dtype dtype, int causal,
                 float softmax_scale, struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  bool empty = false;
  fa_status st = bwd_check_args(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, dtype, softmax_scale, &empty);
  if (st != FA_OK || empty) return st;
  if ((st = check_ptr(workspace, "workspace")) != FA_OK) return st;
  const size_t need = fa::bwd_dense_bytes(B, Hq, Hkv, N, d, causal != 0);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                need);
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, dtype, causal, softmax_scale,
                     stream);
}

// ---- fa_bwd_noalloc: the backward with its workspace in a static device array ----
//
// `scratch` is a file-scope device array: one copy per GPU, created when the code object
// is loaded on that GPU and held until the process ends.  In host code its name is only a
// host-side stand-in, never a device address, so the first call on each device looks up
// that device's copy with hipGetSymbolAddress (with the device current) and keeps the
// pointer; kernels receive only that pointer.  Nothing is allocated or freed per call.
// The backward's workspace needs no clearing: the row-term kernel writes every row term
// and every chunk of a split plan writes its whole partial slot, so the contents a
// previous call left behind are overwritten before they are read.
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fa_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch supports", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(err));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t N, int64_t d, fa_dtype dtype, int causal, float softmax_scale,
                         struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  bool empty = false;
  fa_status st = bwd_check_args(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, dtype, softmax_scale, &empty);
  if (st != FA_OK || empty) return st;
  const size_t need = fa::bwd_dense_bytes(B, Hq, Hkv, N, d, causal != 0);
  if (need > kScratchBytes)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "these sizes need %zu bytes of workspace, more than the %zu bytes of static scratch "
                "fa_bwd_noalloc has; call fa_bwd with a workspace instead",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != FA_OK) return st;
  return bwd_checked(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, N, d, dtype, causal, softmax_scale, stream);
}

size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                                     fa_dtype dtype, int64_t num_splits) {
  bool empty = false;
  if (check_splitkv_sizes(B, Hq, Hkv, Nq, Nk, d, dtype, 0, num_splits, &empty) != FA_OK) return 0;
  if (empty) return 0;
  if (fa::splitkv_is_prefill(Nq, Nk))
    return fa::prefill_workspace_bytes(B, Hq, Nq, d, fa::plan_prefill_split(Nq, num_splits));
  return fa::splitkv_workspace_bytes(B, Hq, Nq, d, fa::plan_splits(B, Hq, Hkv, Nq, Nk, num_splits));
}

int64_t fa_fwd_splitkv_num_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d) {
  bool empty = false;
  if (check_splitkv_sizes(B, Hq, Hkv, Nq, Nk, d, FA_BF16, 0, 0, &empty) != FA_OK || empty) return 0;
  if (fa::splitkv_is_prefill(Nq, Nk)) return fa::plan_prefill_split(Nq, 0).S;
  const fa::SplitPlan p = fa::plan_splits(B, Hq, Hkv, Nq, Nk, 0);
  return (Nk + p.C - 1) / p.C;
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                         int64_t d, fa_dtype dtype, int causal, float softmax_scale, int64_t num_splits,
                         struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  bool empty = false;
  fa_status st = check_splitkv_sizes(B, Hq, Hkv, Nq, Nk, d, dtype, causal, num_splits, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if ((st = check_ptr(q, "q")) != FA_OK || (st = check_ptr(k, "k")) != FA_OK ||
      (st = check_ptr(v, "v")) != FA_OK || (st = check_ptr(o, "o")) != FA_OK ||
      (st = check_ptr(lse, "lse")) != FA_OK || (st = check_ptr(workspace, "workspace")) != FA_OK)
    return st;
  if (fa::splitkv_is_prefill(Nq, Nk)) {   // as many queries as keys: key-split prefill
    const fa::PrefillSplit p = fa::plan_prefill_split(Nq, num_splits);
    const size_t need = fa::prefill_workspace_bytes(B, Hq, Nq, d, p);
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                  need);
    fa::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = (int)B;
    a.Hq = (int)Hq;
    a.Hkv = (int)Hkv;
    a.N = (int)Nq;
    a.Nk = (int)Nk;
    a.maxq = (int)Nq;
    a.maxk = (int)Nk;
    a.wl = -1;
    a.wr = causal ? 0 : -1;
    a.scale = softmax_scale;
    a.scale_log2 = softmax_scale * kLog2e;
    hipError_t err;
    if (p.S == 1) {   // one split: fa_fwd itself (the same bits as the general mode without a mask)
      err = fa::launch_fwd(a, (int)d, dtype == FA_BF16, causal != 0, (hipStream_t)stream);
    } else {
      a.ksplit = p.S;
      a.kchunk = p.C;
      a.opart = static_cast<float*>(workspace);
      a.lpart =
          reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + fa::prefill_opart_bytes(B, Hq, Nq, d, p));
      err = fa::launch_fwd_masked(a, (int)d, dtype == FA_BF16, (hipStream_t)stream);
      if (err == hipSuccess)
        err = fa::launch_lse_combine(a.opart, a.lpart, o, lse, B * Hq * Nq, p.S, (int)d, dtype == FA_BF16,
                                     (hipStream_t)stream);
    }
    if (err != hipSuccess) return fail(FA_ERR_HIP, "key-split forward launch failed: %s", hipGetErrorString(err));
    return FA_OK;
  }
  const fa::SplitPlan p = fa::plan_splits(B, Hq, Hkv, Nq, Nk, num_splits);
  const size_t need = fa::splitkv_workspace_bytes(B, Hq, Nq, d, p);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes,
                need);
  fa::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.opart = static_cast<float*>(workspace);
  a.lpart = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + fa::splitkv_opart_bytes(B, Hq, Nq, d, p));
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.Nq = (int)Nq;
  a.Nk = (int)Nk;
  a.RG = p.RG;
  a.C = p.C;
  a.S4 = p.S4;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t err = fa::launch_splitkv(a, (int)d, dtype == FA_BF16, causal != 0, (hipStream_t)stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "split-KV launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

fa_status fa_lse_combine(const float* o_parts, const float* lse_parts, void* o, float* lse, int64_t rows,
                         int64_t num_parts, int64_t d, fa_dtype dtype, struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  if (rows < 0) return fail(FA_ERR_INVALID_ARGUMENT, "rows must be >= 0 (got %lld)", (long long)rows);
  if (num_parts < 1) return fail(FA_ERR_INVALID_ARGUMENT, "num_parts must be >= 1 (got %lld)", (long long)num_parts);
  if (d < 1) return fail(FA_ERR_INVALID_ARGUMENT, "d must be >= 1 (d=%lld)", (long long)d);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension %lld not supported (64 or 128)",
                                       (long long)d);
  if (dtype != FA_F16 && dtype != FA_BF16) return fail(FA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (num_parts > INT_MAX || rows > (int64_t)INT_MAX * 65536)
    return fail(FA_ERR_INVALID_ARGUMENT, "sizes exceed the supported index range");
  if (rows == 0) return FA_OK;
  fa_status st;
  if ((st = check_ptr(o_parts, "o_parts")) != FA_OK || (st = check_ptr(lse_parts, "lse_parts")) != FA_OK ||
      (st = check_ptr(o, "o")) != FA_OK || (st = check_ptr(lse, "lse")) != FA_OK)
    return st;
  const hipError_t err = fa::launch_lse_combine(o_parts, lse_parts, o, lse, (long long)rows, (int)num_parts, (int)d,
                                                dtype == FA_BF16, (hipStream_t)stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "combine launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

fa_status fa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int64_t max_seqlen_q, int64_t max_seqlen_k,
                        int64_t window_left, int64_t window_right, const int32_t* block_cnt,
                        const int32_t* block_idx, int64_t block_heads, float softmax_scale,
                        struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  bool empty = false;
  fa::FwdArgs a;
  fa_status st = check_masked(B, Hq, Hkv, Nq, Nk, d, dtype, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                              window_left, window_right, softmax_scale, &empty, a);
  if (st != FA_OK) return st;
  if ((st = check_lists(block_cnt, block_idx, block_heads, Hq, empty, a)) != FA_OK || empty) return st;
  if ((st = check_ptr(q, "q")) != FA_OK || (st = check_ptr(o, "o")) != FA_OK || (st = check_ptr(lse, "lse")) != FA_OK)
    return st;
  if (Nk > 0 && ((st = check_ptr(k, "k")) != FA_OK || (st = check_ptr(v, "v")) != FA_OK)) return st;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  const hipError_t err = fa::launch_fwd_masked(a, (int)d, dtype == FA_BF16, (hipStream_t)stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "masked forward launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

size_t fa_bwd_masked_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seqlen_q, int64_t max_seqlen_k,
                                    int block_lists) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || Hq % Hkv != 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return 0;
  if (block_lists) return fa::bwd_list_layout(B, Hq, Hkv, max_seqlen_q, max_seqlen_k).end;
  return fa::bwd_rowterm_bytes(B, Hq, max_seqlen_q);
}

fa_status fa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, fa_dtype dtype,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t max_seqlen_q,
                        int64_t max_seqlen_k, int64_t window_left, int64_t window_right, const int32_t* block_cnt,
                        const int32_t* block_idx, int64_t block_heads, float softmax_scale,
                        struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  bool empty = false;
  fa::BwdArgs a;
  fa_status st = check_masked(B, Hq, Hkv, Nq, Nk, d, dtype, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                              window_left, window_right, softmax_scale, &empty, a);
  if (st != FA_OK) return st;
  if ((st = check_lists(block_cnt, block_idx, block_heads, Hq, empty, a)) != FA_OK || empty) return st;
  const bool lists = block_idx != nullptr;
  // run records: two ints per (query head of a group, 256-query block), G below 2^20
  if (lists && (Hq / Hkv >= (1 << 20) || fa::bwd_runs_stride(Hq, Hkv, a.maxq) >= (1LL << 30)))
    return fail(FA_ERR_UNSUPPORTED, "block lists: Hq/Hkv * ceil(max_seqlen_q/256) too large for the backward");
  if ((st = check_ptr(q, "q")) != FA_OK || (st = check_ptr(o, "o")) != FA_OK || (st = check_ptr(lse, "lse")) != FA_OK ||
      (st = check_ptr(dout, "dout")) != FA_OK || (st = check_ptr(dq, "dq")) != FA_OK ||
      (st = check_ptr(workspace, "workspace")) != FA_OK)
    return st;
  if (Nk > 0 && ((st = check_ptr(k, "k")) != FA_OK || (st = check_ptr(v, "v")) != FA_OK ||
                 (st = check_ptr(dk, "dk")) != FA_OK || (st = check_ptr(dv, "dv")) != FA_OK))
    return st;
  const fa::BwdListLayout lay = fa::bwd_list_layout(B, Hq, Hkv, a.maxq, a.maxk);
  const size_t need = lists ? lay.end : fa::bwd_rowterm_bytes(B, Hq, a.maxq);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  if (lists) {
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    a.runs = reinterpret_cast<int*>(ws + lay.runs);
    a.rstride = fa::bwd_runs_stride(Hq, Hkv, a.maxq);
    a.plan = reinterpret_cast<int*>(ws + lay.plan);
    a.table = reinterpret_cast<int*>(ws + lay.table);
    a.pool = reinterpret_cast<float*>(ws + lay.pool);
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.rowterm = static_cast<float*>(workspace);
  const hipError_t err = fa::launch_bwd_masked(a, (int)d, dtype == FA_BF16, (hipStream_t)stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "masked backward launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

size_t fa_fp8_v_codes_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return 0;
  return (size_t)(B * H * ((N + 63) / 64) * d * 64);
}

fa_status fa_fp8_quantize_rows(const void* x, const float* signs, void* codes, float* scales, int64_t B,
                               int64_t H, int64_t N, int64_t d, fa_dtype dtype, int64_t block_rows,
                               struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  return run_fp8_quant(x, signs, codes, scales, B, H, N, d, dtype, block_rows, signs ? 0 : 1, (hipStream_t)stream);
}

fa_status fa_fp8_quantize_v(const void* x, void* codes, float* scales, int64_t B, int64_t H, int64_t N, int64_t d,
                            fa_dtype dtype, int64_t block_rows, struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  return run_fp8_quant(x, nullptr, codes, scales, B, H, N, d, dtype, block_rows, 2, (hipStream_t)stream);
}

fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scales, const float* k_scales,
                     const float* v_scales, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                     int64_t d, int64_t block_q, int64_t block_kv, int causal, float softmax_scale,
                     struct ihipStream_t* stream) {
  g_last_error[0] = '\0';
  bool empty = false;
  fa_status st = check_sizes(B, Hq, Hkv, N, d, FA_BF16, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(softmax_scale)) != FA_OK) return st;
  if (!fp8_block_ok(block_q) || !fp8_block_ok(block_kv))
    return fail(FA_ERR_INVALID_ARGUMENT, "block_q and block_kv must be 64, 128 or 256 (got %lld, %lld)",
                (long long)block_q, (long long)block_kv);
  if (empty) return FA_OK;
  if ((st = check_ptr(q8, "q8")) != FA_OK || (st = check_ptr(k8, "k8")) != FA_OK ||
      (st = check_ptr(v8, "v8")) != FA_OK || (st = check_ptr4(q_scales, "q_scales")) != FA_OK ||
      (st = check_ptr4(k_scales, "k_scales")) != FA_OK || (st = check_ptr4(v_scales, "v_scales")) != FA_OK ||
      (st = check_ptr(o, "o")) != FA_OK || (st = check_ptr(lse, "lse")) != FA_OK)
    return st;
  fa::Fp8FwdArgs a;
  a.q = static_cast<const uint8_t*>(q8);
  a.k = static_cast<const uint8_t*>(k8);
  a.v = static_cast<const uint8_t*>(v8);
  a.qs = q_scales;
  a.ks = k_scales;
  a.vs = v_scales;
  a.o = o;
  a.lse = lse;
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.N = (int)N;
  a.qshift = log2_block(block_q);
  a.kvshift = log2_block(block_kv);
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t err = fa::launch_fwd_fp8(a, (int)d, causal != 0, (hipStream_t)stream);
  if (err != hipSuccess) return fail(FA_ERR_HIP, "FP8 forward launch failed: %s", hipGetErrorString(err));
  return FA_OK;
}

}  // extern "C"
