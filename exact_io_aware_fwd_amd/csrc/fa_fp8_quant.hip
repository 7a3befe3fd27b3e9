// Block quantisation to FP8 (e4m3) for the FP8 forward pass, with the optional
// random-sign Hadamard transform of queries and keys.
//
// Method: "Flash Attention" (wiki), section "FlashAttention-3" — block quantization
// plus incoherent processing (random signs and a Hadamard transform, the same
// orthogonal transform for queries and keys, so their dot products are unchanged);
// "FlashAttention" (explainer), section "What Hopper bought FlashAttention-3" —
// per-block scaling.
//
// Definition implemented (the readings where the pages are silent):
//  * x -> x M with M = diag(sigma) H_d / sqrt(d), H_d the Sylvester Hadamard matrix.
//    x diag(sigma) H_d is a signed sum of half-precision values and is formed exactly
//    in fp64 (a fast Walsh-Hadamard transform: log2 d butterfly stages); the
//    normalisation is one fp64 multiplication by the fp64 value nearest 1/sqrt(d); the
//    result is rounded to fp32 (round to nearest even).
//  * A block is `block_rows` consecutive rows of one head.  Its scale is 2^e with e the
//    smallest integer such that the block's largest |value| is at most 448 * 2^e
//    (e = 0 for an all-zero block, clamped to [-127, 127]); the codes are
//    e4m3(value * 2^-e), round to nearest even (v_cvt_pk_fp8_f32).  Scaling by a power
//    of two is exact, so every code is decided by one rounding of an fp32 value.
//
// gfx950 design.  One workgroup per scale block (block_rows * d / 64 threads), two rows
// per thread and 32 consecutive columns per thread (four 16-byte loads); five butterfly
// stages run inside the thread and the d/32 threads of a row are lanes of one quad, so
// the remaining one or two stages are DPP quad permutations (no LDS traffic).  The
// values stay in registers between the block maximum and the encoding (one HBM read).
//  * Query/key codes keep the input layout [B, H, N, d].
//  * Value codes are written in the layout the forward pass feeds to the matrix core:
//    per 64-key tile a transposed [d][64] byte block, [B, H, ceil(N/64), d, 64], with
//    the keys of a tile permuted so that each lane's 32-byte operand is contiguous
//    (position 32h + 16t + 4a + b holds key 32t + 8a + 4h + b, matching the order in
//    which the score layout hands the probabilities to the product).  Keys past N are
//    written as code 0.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// e = smallest integer with amax <= 448 * 2^e.  448 = 0.875 * 2^9, so for
// amax = m * 2^E with m in [0.5, 1): e = E - 9, plus one when m > 0.875.
static __device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t bits = __float_as_uint(amax);
  if (bits < 0x00800000u) return -127;                 // fp32 subnormal: far below 448 * 2^-127
  const int E = (int)(bits >> 23) - 126;               // amax = m * 2^E, m = 1.f * 2^-1 ...
  const uint32_t man = bits & 0x007FFFFFu;             // m = (1 + man / 2^23) / 2
  int e = E - 9 + (man > 0x00600000u ? 1 : 0);         // m > 0.875  <=>  man > 0.75 * 2^23
  return min(max(e, -127), 127);
}

// 2^e as fp32 for e in [-127, 127] (2^-127 is subnormal).
static __device__ __forceinline__ float pow2f(int e) {
  return e >= -126 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// Lane exchange within quads for the butterflies across threads: lane l receives the
// value of lane l ^ M (M = 1 or 2), one DPP move per 32-bit half.
template <int M>
static __device__ __forceinline__ double quad_xor(double x) {
  constexpr int ctrl = M == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, ctrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), ctrl, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

template <class Tag, int D, bool ROT, bool VT>
__global__ void __launch_bounds__(512) fp8_quant_kernel(const QuantArgs a) {
  using E = Elt<Tag>;
  constexpr int TPR = D / 32;        // threads per row (32 consecutive columns each)
  constexpr int NP = 2;              // rows per thread
  const int t = threadIdx.x;
  const int nt = blockDim.x;         // block_rows * D / 64
  const int rpp = nt / TPR;          // rows per pass
  const int j = t % TPR;
  const int r0 = t / TPR;
  const int bh = blockIdx.x / a.nblk;
  const int blk = blockIdx.x - bh * a.nblk;
  const int row0 = blk * a.block_rows;
  const uint16_t* X = (const uint16_t*)a.x + (size_t)bh * a.N * D;

  uint32_t negm = 0;                 // bit i: column 32j + i has sign -1
  if constexpr (ROT) {
#pragma unroll
    for (int i = 0; i < 32; ++i) negm |= (a.signs[32 * j + i] < 0.f ? 1u : 0u) << i;
  }

  float y[NP][32];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = row0 + p * rpp + r0;
    u32x4 raw[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    if (row < a.N) {
      const u32x4* src = (const u32x4*)(X + (size_t)row * D + 32 * j);
#pragma unroll
      for (int c = 0; c < 4; ++c) raw[c] = src[c];
    }
    float f[32];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * c + 2 * i] = E::to_f32((uint16_t)(raw[c][i] & 0xFFFFu));
        f[8 * c + 2 * i + 1] = E::to_f32((uint16_t)(raw[c][i] >> 16));
      }
    if constexpr (ROT) {
      double z[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) z[i] = (double)((negm >> i) & 1u ? -f[i] : f[i]);
      // butterflies over the five index bits inside the thread ...
#pragma unroll
      for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (!(i & h)) {
            const double u = z[i], w = z[i + h];
            z[i] = u + w;
            z[i + h] = u - w;
          }
      // ... and over the bits that select the thread: the lower index keeps u + w, the
      // upper gets u - w = o - z (o the partner's value); all sums are exact
      if constexpr (TPR >= 2) {
        const double s1 = (j & 1) ? -1.0 : 1.0;
#pragma unroll
        for (int i = 0; i < 32; ++i) z[i] = fma(s1, z[i], quad_xor<1>(z[i]));
      }
      if constexpr (TPR >= 4) {
        const double s2 = (j & 2) ? -1.0 : 1.0;
#pragma unroll
        for (int i = 0; i < 32; ++i) z[i] = fma(s2, z[i], quad_xor<2>(z[i]));
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) y[p][i] = (float)(z[i] * a.inv_sqrt_d);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) y[p][i] = f[i];
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[p][i]));
  }

  // block maximum: lanes, then waves through LDS
  __shared__ float red[8];
  __shared__ int eblk;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  if (t == 0) {
    float mx = red[0];
    for (int w = 1; w < nt / 64; ++w) mx = fmaxf(mx, red[w]);
    const int e = block_exponent(mx);
    eblk = e;
    a.scales[(size_t)bh * a.nblk + blk] = pow2f(e);
  }
  __syncthreads();
  const float inv = pow2f(-eblk);     // -e in [-127, 127]; e <= 126 for finite fp32 data

  uint32_t code[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[p][4 * h] * inv, y[p][4 * h + 1] * inv, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(y[p][4 * h + 2] * inv, y[p][4 * h + 3] * inv, w, true);
      code[p][h] = (uint32_t)w;
    }

  if constexpr (!VT) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = row0 + p * rpp + r0;
      if (row < a.N) {
        u32x4* dst = (u32x4*)(a.codes + ((size_t)bh * a.N + row) * D + 32 * j);
        dst[0] = u32x4{code[p][0], code[p][1], code[p][2], code[p][3]};
        dst[1] = u32x4{code[p][4], code[p][5], code[p][6], code[p][7]};
      }
    }
  } else {
    // transpose through LDS: the block's codes as [row][d] bytes, then 16-byte segments
    // of the [d][64] tiles, each gathered from one column
    __shared__ __attribute__((aligned(16))) unsigned char tileb[256 * D];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      u32x4* dst = (u32x4*)(tileb + (p * rpp + r0) * D + 32 * j);
      dst[0] = u32x4{code[p][0], code[p][1], code[p][2], code[p][3]};
      dst[1] = u32x4{code[p][4], code[p][5], code[p][6], code[p][7]};
    }
    __syncthreads();
    const int nkb = (a.N + 63) / 64;
#pragma unroll
    for (int sgi = 0; sgi < 4; ++sgi) {
      const int s = t + sgi * nt;           // segment: tile kt, row d, quarter qq
      const int kt = s / (4 * D);
      const int d = (s / 4) % D;
      const int qq = s & 3;
      const int tile = row0 / 64 + kt;
      if (tile >= nkb) continue;
      const int half = qq >> 1, tt = qq & 1;
      uint32_t w[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {         // bytes 4g .. 4g+3: keys 32tt + 8g + 4half + 0..3
        const int key = 64 * kt + 32 * tt + 8 * g + 4 * half;
        w[g] = (uint32_t)tileb[key * D + d] | ((uint32_t)tileb[(key + 1) * D + d] << 8) |
               ((uint32_t)tileb[(key + 2) * D + d] << 16) | ((uint32_t)tileb[(key + 3) * D + d] << 24);
      }
      *(u32x4*)(a.codes + (((size_t)bh * nkb + tile) * D + d) * 64 + 16 * qq) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

template <class Tag, int D>
static hipError_t launch_quant_t(const QuantArgs& a, int mode, hipStream_t stream) {
  const long long nblocks = (long long)a.BH * a.nblk;
  if (nblocks <= 0) return hipSuccess;
  const int nt = a.block_rows * D / 64;
  if (mode == 0) hipLaunchKernelGGL((fp8_quant_kernel<Tag, D, true, false>), dim3((unsigned)nblocks), dim3(nt), 0, stream, a);
  else if (mode == 1) hipLaunchKernelGGL((fp8_quant_kernel<Tag, D, false, false>), dim3((unsigned)nblocks), dim3(nt), 0, stream, a);
  else hipLaunchKernelGGL((fp8_quant_kernel<Tag, D, false, true>), dim3((unsigned)nblocks), dim3(nt), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fp8_quant(const QuantArgs& a, int d, bool bf16, int mode, hipStream_t stream) {
  if (bf16) return d == 128 ? launch_quant_t<bf16_tag, 128>(a, mode, stream) : launch_quant_t<bf16_tag, 64>(a, mode, stream);
  return d == 128 ? launch_quant_t<f16_tag, 128>(a, mode, stream) : launch_quant_t<f16_tag, 64>(a, mode, stream);
}

}  // namespace fa
