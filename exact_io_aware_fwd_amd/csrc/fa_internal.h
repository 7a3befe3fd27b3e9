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
};

// Return a hipError_t from the launches (hipSuccess when all were enqueued).
hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16, bool causal, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16, bool causal, hipStream_t stream);

// Workspace of the backward pass: two fp32 row terms per query row, rows padded to a
// multiple of 32 per head (256 bytes per 32-row block).
inline size_t bwd_rowterm_bytes(int64_t B, int64_t Hq, int64_t N) {
  return (size_t)(B * Hq * ((N + 31) / 32) * 256);
}

}  // namespace fa
