// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// element traits with the 32x32x16 MFMA, packed round-to-nearest-even
// conversions, the LDS transposing read, and wave-level reductions.
//
// MFMA v_mfma_f32_32x32x16_{bf16,f16} lane layout (wave64), checked on the device:
//   A (32x16):  lane l holds A[l%32][8*(l/32) + 0..7]
//   B (16x32):  lane l holds B[8*(l/32) + 0..7][l%32]
//   C (32x32):  lane l holds C[8*(v/4) + 4*(l/32) + v%4][l%32], v = 0..15
// ds_read_b64_tr_b16: within each 16-lane group, with M[j][c] the four 16-bit
// elements lane j addresses, lane i receives M[4r + i/4][i%4] for r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct bf16_tag {};
struct f16_tag {};

template <class Tag> struct Elt;

template <> struct Elt<bf16_tag> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two floats -> two bf16 (RNE) in one dword, `lo` in the low half
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    return __uint_as_float(((uint32_t)bits) << 16);
  }
};

template <> struct Elt<f16_tag> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
};

// MFMA accumulation into an accumulator held in AGPRs for its whole life (inline asm:
// the "a" constraint keeps the compiler from moving it between register files).  The
// compiler does not see these MFMAs, so their hazards are covered by hand:
//   - VALU write of a B operand -> MFMA read needs 2 wait states: mma_acc_fresh
//     issues s_nop 1 first; use it for the first MFMA after packing an operand;
//   - accumulator init (VALU) -> first MFMA: acc_init ends with s_nop 1;
//   - MFMA write -> VALU read of the accumulator: acc_drain waits 32 cycles.
// Back-to-back MFMAs on the same accumulator need no wait states (hardware forwarding),
// and LDS loads feeding the A operand are covered by the compiler's s_waitcnt.
template <class Tag> struct AccMma;
template <> struct AccMma<bf16_tag> {
  static __device__ __forceinline__ void mma(f32x16& acc, u32x4 a, u32x4 b) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
#endif
  }
  static __device__ __forceinline__ void mma_fresh(f32x16& acc, u32x4 a, u32x4 b) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
#endif
  }
};
template <> struct AccMma<f16_tag> {
  static __device__ __forceinline__ void mma(f32x16& acc, u32x4 a, u32x4 b) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
#endif
  }
  static __device__ __forceinline__ void mma_fresh(f32x16& acc, u32x4 a, u32x4 b) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
#endif
  }
};
template <int N>
static __device__ __forceinline__ void acc_init(f32x16 (&acc)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+a"(acc[i]));
#endif
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 1");
#endif
}
template <int N>
static __device__ __forceinline__ void acc_drain(f32x16 (&acc)[N]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_nop 15\n\ts_nop 15");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(acc[i]));
#endif
}

static __device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 8 contiguous bytes of LDS, read transposed across each 16-lane group.
static __device__ __forceinline__ u32x2 lds_read_tr(const unsigned char* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

static __device__ __forceinline__ u32x4 cat(u32x2 lo, u32x2 hi) {
  u32x4 r = {lo.x, lo.y, hi.x, hi.y};
  return r;
}

// Reductions across the two half-waves: every lane gets op(x[l], x[l^32]).
// permlane32_swap(x, x) yields (x[l], x[l+32]) in lanes 0-31 and (x[l-32], x[l]) in 32-63.
static __device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
static __device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

static __device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Write one row of a transposed accumulator (x^T in NE 32x32 MFMA C tiles: this lane holds
// elements 32e + 8g + 4hh + 0..3 of its row, g = 0..3), times `mul`, rounded to the element
// type, 16 bytes a lane.  Of each pair of 8-element chunks 32e + 16m and 32e + 16m + 8, the
// lane with hh = 0 writes the first (its own 4 elements, then its partner's) and the lane
// with hh = 1 the second; the partners (lanes l and l + 32, the same row) swap one 8-byte
// piece with permlane32_swap.  Both partners must take this call together (they share the
// row, so a row bound keeps them in step).
template <class E, int NE>
static __device__ __forceinline__ void store_row16(unsigned char* row, const f32x16 (&x)[NE], float mul, int hh) {
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint32_t w[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int g = 2 * m + t;
        w[t][0] = E::pack(x[e][4 * g + 0] * mul, x[e][4 * g + 1] * mul);
        w[t][1] = E::pack(x[e][4 * g + 2] * mul, x[e][4 * g + 3] * mul);
      }
      uint32_t y[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t send = hh ? w[0][j] : w[1][j];
        const auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
        y[j] = hh ? r[0] : r[1];
      }
      const u32x4 out = hh ? u32x4{y[0], y[1], w[1][0], w[1][1]} : u32x4{w[0][0], w[0][1], y[0], y[1]};
      *(u32x4*)(row + (32 * e + 16 * m + 8 * hh) * 2) = out;
    }
}

// Smallest p in [0, n) with list[p] >= t (n if none); list ascending (block lists).
static __device__ __forceinline__ int lower_bound_tiles(const int* list, int n, int t) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list[mid] < t) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// s_waitcnt vmcnt(0): this wave's global and buffer loads (LDS DMA included) are done.
// A workgroup barrier does not wait for them by itself; put this before the barrier
// that publishes a tile loaded by several waves.  (The builtin, unlike inline asm, is
// seen by the compiler's wait-count bookkeeping.)
static __device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Compiler fences on values (device pass only; the host pass never sees VGPR constraints).
// opaque(x): x is redefined here, so nothing computed from it is hoisted above this point.
// keep(x):   x must be computed before this point (no sinking into later blocks).
template <class T>
static __device__ __forceinline__ void opaque(T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
}
template <class T>
static __device__ __forceinline__ void keep(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

static constexpr float kLog2e = 1.4426950408889634f;
static constexpr float kLn2 = 0.6931471805599453f;

}  // namespace fa
