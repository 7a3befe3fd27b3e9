// FP8 (e4m3) forward pass of attention for gfx950: both products on the FP8 matrix
// core, online softmax in fp32, O (bf16) and LSE (fp32) out.
//
// Method: "Flash Attention" (wiki), section "FlashAttention-3", and "FlashAttention"
// (explainer), section "What Hopper bought FlashAttention-3": FP8 operands with
// per-block scales, queries and keys taken through the random-sign Hadamard transform
// beforehand (the quantiser in fa_fp8_quant.hip).  The tiling and the online softmax are the forward pass of
// "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section
// "FlashAttention-1: tiling plus online softmax", with the work split of its
// "FlashAttention-2" section and the conditional rescaling of its "FlashAttention-4"
// section.  The probabilities are rounded to e4m3 for the second product (values up
// to 2^8 thanks to the rescaling threshold, well inside the format's 448); the row
// sums that give the LSE use the unrounded fp32 probabilities.
//
// gfx950 design.
//  * v_mfma_scale_f32_32x32x64_f8f6f4: A and B pair byte for byte per lane (lane l
//    holds row l % 32 and one 32-value half of the 64-long product, half l / 32), C is
//    laid out as in the 16-bit 32x32 products, and each lane's 8-bit power-of-two scale
//    multiplies its own 32 values.  The block scales of Q, K and V are those scale
//    operands, so dequantisation costs no instruction.
//  * Scores are formed transposed, S^T = K Q^T (lane = query), 64 keys per unit: two
//    32x32 score tiles per unit, d/64 products each.  The probabilities of both tiles
//    are exactly one B operand of O^T += V^T P^T (64 keys), in the key order the
//    quantiser used for the value tiles, so the value operand is a plain 32-byte row
//    read and P never leaves the registers.
//  * A workgroup owns 256 queries (8 waves x 32); K and V tiles (64 keys) go from HBM
//    into LDS by buffer loads to LDS, four slots, three tiles ahead.  Row pitches
//    d+16 bytes (K) and 80 bytes (V^T) keep 16 lanes reading 16 bytes from 16
//    consecutive rows on distinct banks.
//  * As in the 16-bit forward pass: the products of unit u+1 are issued during the
//    softmax of unit u, the two waves of a SIMD run half a unit apart (the late group
//    forms its scores before the tile barrier, which is why it needs tile u+1 one
//    barrier earlier and hence the fourth slot), the reference max moves only by more
//    than 8 (log2 units), and O is rescaled only when a lane of the wave moved it.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

static __device__ __forceinline__ f32x16 mma_fp8(u32x8 a, u32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b), c,
                                                         0, 0, 0, sa, 0, sb);
}

// E8M0 exponent of a power-of-two fp32 scale (2^-127 is the subnormal 0x00400000 -> 0).
static __device__ __forceinline__ int e8m0(float s) { return (int)(__float_as_uint(s) >> 23); }

// HBM -> LDS of tile t: K rows [64t, 64t+64) (d bytes each, pitch d+16 in LDS) and the
// value tile t (d rows of 64 bytes, pitch 80).  Load i of this wave covers slot bytes
// [1024n, 1024n+1024), n = wave + 8i; doff[i] is the lane's source byte.  The K
// descriptor ends at row N, so rows past the end arrive as zeros.  (A device function,
// not a lambda: the buffer builtins exist only for the device.)
template <int D, int IPW>
static __device__ __forceinline__ void fp8_tile_load(const unsigned char* Kg, const unsigned char* Vg, int N, int t,
                                                     int wave, const int* doff, unsigned char* sl) {
  constexpr int KI = 64 * (D + 16) / 1024;
  constexpr int NI = KI + D * 80 / 1024;
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + (size_t)t * 64 * D), (short)0, (N - t * 64) * D, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + (size_t)t * 64 * D), (short)0, 64 * D, 0x00020000);
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int n = wave + 8 * i;
    if (n < KI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lvoid*)(sl + n * 1024), 16, doff[i], 0, 0, 0);
    else if (n < NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lvoid*)(sl + n * 1024), 16, doff[i], 0, 0, 0);
  }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512) fwd_fp8_kernel(const Fp8FwdArgs a) {
  using E = Elt<bf16_tag>;
  constexpr int NW = 8;                 // waves per workgroup
  constexpr int BR = 32 * NW;           // query rows per workgroup
  constexpr int BC = 64;                // keys per unit (one tile)
  constexpr int KP = D + 16;            // LDS pitch of K rows
  constexpr int VP = 80;                // LDS pitch of V^T rows (64 keys + 16)
  constexpr int KBYTES = 64 * KP;
  constexpr int VBYTES = D * VP;
  constexpr int SLOT = KBYTES + VBYTES;
  constexpr int KI = KBYTES / 1024;     // 1024-byte wave loads per K tile
  constexpr int NI = SLOT / 1024;
  constexpr int IPW = (NI + NW - 1) / NW;
  constexpr int NC = D / 64;            // products per score tile
  constexpr int NSL = 2 * NC;           // score products per unit
  constexpr int NE = D / 32;            // 32-row blocks of O^T
  constexpr int EPS = 32 / NSL;         // exponentials per score product
  constexpr int PD = 2;                 // LDS read-ahead, in products
  constexpr float TAU = 8.f;
  static_assert(KBYTES % 1024 == 0 && VBYTES % 1024 == 0, "tiles are whole wave loads");
  static_assert(NW == 8 && KI == 64 * (D + 16) / 1024 && NI == KI + D * 80 / 1024, "fp8_tile_load's layout");
  static_assert(PD <= NSL && PD <= NE, "read-ahead within one phase");

  __shared__ __attribute__((aligned(1024))) unsigned char slot0[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot3[SLOT];
  auto slot = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? slot0 : i == 1 ? slot1 : i == 2 ? slot2 : slot3;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;

  int b, hq, iq;
  map_q_block((N + BR - 1) / BR, a.B, a.Hq, a.Hkv, b, hq, iq);
  const int hkv = hq / (a.Hq / a.Hkv);
  const int nkb = (N + BC - 1) / BC;
  const size_t qhead = (size_t)(b * a.Hq + hq) * (size_t)N;
  const size_t kvh = (size_t)(b * a.Hkv + hkv);
  const unsigned char* Qg = a.q + qhead * D;
  const unsigned char* Kg = a.k + kvh * (size_t)N * D;
  const unsigned char* Vg = a.v + kvh * (size_t)nkb * (BC * D);
  const int nqblk = (N + (1 << a.qshift) - 1) >> a.qshift;
  const int nkvblk = (N + (1 << a.kvshift) - 1) >> a.kvshift;
  const float* ksh = a.ks + kvh * nkvblk;
  const float* vsh = a.vs + kvh * nkvblk;

  const int q0 = iq * BR;
  const int qw = q0 + wave * 32;
  const int myq = qw + r32;

  // Q^T as the B operand: lane holds Q[myq][64c + 32hh .. +31], with its block's scale
  u32x8 qf[NC];
  int sq = 127;
  if (myq < N) {
    const unsigned char* qp = Qg + (size_t)myq * D + 32 * hh;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x4 lo = *(const u32x4*)(qp + 64 * c), hi = *(const u32x4*)(qp + 64 * c + 16);
      qf[c] = u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    sq = e8m0(a.qs[(size_t)(b * a.Hq + hq) * nqblk + (myq >> a.qshift)]);
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = u32x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  auto kscale = [&](int u) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(e8m0(ksh[(u * BC) >> a.kvshift]));
  };
  auto vscale = [&](int u) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(e8m0(vsh[(u * BC) >> a.kvshift]));
  };

  const int ntile = CAUSAL ? min(nkb, (min(q0 + BR, N) - 1) / BC + 1) : nkb;

  // ---- HBM -> LDS: tile t of K (rows of d bytes) and V^T (d rows of 64 bytes) ----
  // Lane's 16 bytes of load i land at slot byte 1024 n + 16 lane (n = wave + NW i);
  // lanes that land on row padding fetch byte 0 again.
  int doff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int n = wave + NW * i;
    if (n < KI) {
      const int o = n * 1024 + lane * 16, row = o / KP, col = o - row * KP;
      doff[i] = col < D ? row * D + col : 0;
    } else {
      const int o = (n - KI) * 1024 + lane * 16, row = o / VP, col = o - row * VP;
      doff[i] = col < 64 ? row * 64 + col : 0;
    }
  }
  auto dma = [&](int t, unsigned char* sl) __attribute__((always_inline)) {
    fp8_tile_load<D, IPW>(Kg, Vg, N, t, wave, doff, sl);
  };

  // K fragment of score product k (tile k / NC, chunk k % NC); V fragment of O^T block e
  auto kread = [&](const unsigned char* sl, int k) __attribute__((always_inline)) {
    const unsigned char* p = sl + (32 * (k / NC) + r32) * KP + 64 * (k % NC) + 32 * hh;
    const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
    return u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };
  auto vread = [&](const unsigned char* sl, int e) __attribute__((always_inline)) {
    const unsigned char* p = sl + KBYTES + (32 * e + r32) * VP + 32 * hh;
    const u32x4 lo = *(const u32x4*)p, hi = *(const u32x4*)(p + 16);
    return u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };

  const float c2 = a.scale_log2;
  float mr = -INFINITY;
  float l_run = 0.f;
  f32x16 o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e] = zero16();

  auto newref = [&](float mx, bool& raise, float& mref) __attribute__((always_inline)) {
    mx *= c2;
    raise = mx > mr + TAU;
    const float mnew = raise ? mx : mr;
    const float alpha = (mr == -INFINITY) ? 0.f : fast_exp2(mr - mnew);
    mref = (mnew == -INFINITY) ? 0.f : mnew;
    mr = mnew;
    return alpha;
  };
  // keys past N, or (causal) after the query, to -inf: score v of tile t is key
  // 64u + 32t + 8(v/4) + 4hh + v%4
  auto mask_unit = [&](int u, f32x16 (&s)[2]) __attribute__((always_inline)) {
    int lim = N - u * BC - 4 * hh;
    if (CAUSAL) lim = min(lim, myq - u * BC - 4 * hh + 1);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * t + 8 * (v >> 2) + (v & 3) >= lim) s[t][v] = -INFINITY;
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[e][v] *= alpha;
  };

  struct Ref {
    float mref;
    float alpha;
    bool raise;
  };

  // S-phase of unit u.  First O is rescaled if unit u moved the reference (a branch at
  // the start, so that nothing issued later in the phase is sunk past it).  Then NSL
  // slots, each with EPS of unit u's exponentials (and their row-sum adds) followed by
  // one score product of unit u+1 (K from sln, read PD slots ahead, the first ones at
  // the start of the phase, so the exponentials cover the LDS latency).  Ends with P
  // packed to e4m3, the B operand of the value products.
  auto sphase = [&](const unsigned char* sln, f32x16 (&sc)[2], f32x16 (&sn)[2], int skn, const Ref& rf,
                    float& rs) __attribute__((always_inline)) -> u32x8 {
    if (__builtin_amdgcn_ballot_w64(rf.raise) != 0) rescale(rf.alpha);
    u32x8 kf[NSL];
#pragma unroll
    for (int i = 0; i < PD; ++i) kf[i] = kread(sln, i);
#pragma unroll
    for (int k = 0; k < NSL; ++k) {
      if (k + PD < NSL) kf[k + PD] = kread(sln, k + PD);
#pragma unroll
      for (int x = k * EPS; x < (k + 1) * EPS; ++x) {
        const float p = fast_exp2(fmaf(sc[x >> 4][x & 15], c2, -rf.mref));
        sc[x >> 4][x & 15] = p;
        rs += p;
      }
      keep(rs);
      const int t = k / NC, c = k % NC;
      sn[t] = mma_fp8(kf[k], qf[c], c == 0 ? zero16() : sn[t], skn, sq);
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t w[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(sc[t][4 * g], sc[t][4 * g + 1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(sc[t][4 * g + 2], sc[t][4 * g + 3], x, true);
        w[4 * t + g] = (uint32_t)x;
      }
    const u32x8 pf = u32x8{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
    keep(pf);
    __builtin_amdgcn_sched_barrier(0);
    return pf;
  };
  // PV-phase of unit u: NE slots, each one value product (V from slc, read PD slots
  // ahead) after a share of the row max of unit u+1 (masked under MASK): tile 0's
  // scores in the first slot, tile 1's (the last product of the S-phase) in the second,
  // the new reference in the third (the second for d = 64).
  auto pphase = [&](auto MASK, int u, const unsigned char* slc, f32x16 (&sn)[2], int svc, Ref& rf,
                    const u32x8& pf) __attribute__((always_inline)) {
    u32x8 vf[NE];
#pragma unroll
    for (int i = 0; i < PD; ++i) vf[i] = vread(slc, i);
    float mx = 0.f;
    if constexpr (decltype(MASK)::value) mask_unit(u + 1, sn);
#pragma unroll
    for (int k = 0; k < NE; ++k) {
      if (k + PD < NE) vf[k + PD] = vread(slc, k + PD);
      if (k == 0) {
        mx = sn[0][0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sn[0][v]);
        keep(mx);
      }
      if (k == 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sn[1][v]);
        mx = half_max(mx);
        keep(mx);
        if constexpr (NE == 2) {
          rf.alpha = newref(mx, rf.raise, rf.mref);
          keep(rf.alpha);
          keep(rf.mref);
        }
      }
      if (NE > 2 && k == 2) {
        rf.alpha = newref(mx, rf.raise, rf.mref);
        keep(rf.alpha);
        keep(rf.mref);
      }
      o[k] = mma_fp8(vf[k], pf, o[k], svc, 127);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 sa[2], sb[2];
  Ref rf;
  // Unit u in slot T = u % 4: [late group: S-phase] barrier, load tile u+3, [early group:
  // S-phase], PV-phase.  Scores alternate between sa (even u) and sb (odd u).
  auto unit = [&](auto Tc, auto MASK, auto LATE, int u) __attribute__((always_inline)) {
    constexpr int T = decltype(Tc)::value;
    unsigned char* const sc = slot(T);
    unsigned char* const sn = slot((T + 1) % 4);
    f32x16(&cur)[2] = (T % 2 == 0) ? sa : sb;
    f32x16(&nxt)[2] = (T % 2 == 0) ? sb : sa;
    const int skn = kscale(min(u + 1, ntile - 1));
    const int svc = vscale(u);
    const float alpha = rf.alpha;
    float rs = 0.f;
    u32x8 pf;
    if constexpr (decltype(LATE)::value) pf = sphase(sn, cur, nxt, skn, rf, rs);
    if (u > 0) {
      wait_loads();
      __syncthreads();
    }
    if (u + 3 < ntile) dma(u + 3, slot((T + 3) % 4));
    if constexpr (!decltype(LATE)::value) pf = sphase(sn, cur, nxt, skn, rf, rs);
    pphase(MASK, u, sc, nxt, svc, rf, pf);
    l_run = fmaf(l_run, alpha, rs);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using Plain = std::false_type;
  using Masked = std::true_type;

  dma(0, slot0);
  if (ntile > 1) dma(1, slot1);
  if (ntile > 2) dma(2, slot2);
  wait_loads();
  __syncthreads();
  {
    const int sk0 = kscale(0);
#pragma unroll
    for (int k = 0; k < NSL; ++k) {
      const int t = k / NC, c = k % NC;
      sa[t] = mma_fp8(kread(slot0, k), qf[c], c == 0 ? zero16() : sa[t], sk0, sq);
    }
  }
  mask_unit(0, sa);
  {
    float mx = sa[0][0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sa[0][v]);
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sa[1][v]);
    rf.alpha = newref(half_max(mx), rf.raise, rf.mref);
  }
  // Units whose successor precedes every wave's first masked unit (the one holding the
  // diagonal of the workgroup's first rows when causal, or the last key) need no mask.
  const int ulast0 = (CAUSAL ? min(q0 + 31, N - 1) : N - 1) / BC;
  const int J1 = min(ntile, max(ulast0 - 1, 0)) / 4 * 4;
  auto run = [&](auto LATE) __attribute__((always_inline)) {
    int u = 0;
    for (; u < J1; u += 4) {
      unit(I0{}, Plain{}, LATE, u);
      unit(I1{}, Plain{}, LATE, u + 1);
      unit(I2{}, Plain{}, LATE, u + 2);
      unit(I3{}, Plain{}, LATE, u + 3);
    }
    for (; u < ntile; u += 4) {
      unit(I0{}, Masked{}, LATE, u);
      if (u + 1 >= ntile) break;
      unit(I1{}, Masked{}, LATE, u + 1);
      if (u + 2 >= ntile) break;
      unit(I2{}, Masked{}, LATE, u + 2);
      if (u + 3 >= ntile) break;
      unit(I3{}, Masked{}, LATE, u + 3);
    }
  };
  if (wave >= NW / 2) run(std::true_type{});
  else run(std::false_type{});

  const float l_tot = half_sum(l_run);
  if (myq < N) {
    const float inv = 1.f / l_tot;
    store_row16<E>((unsigned char*)a.o + (qhead + myq) * (size_t)(2 * D), o, inv, hh);
    if (hh == 0) a.lse[qhead + myq] = (mr + log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_fp8_t(const Fp8FwdArgs& a, hipStream_t stream) {
  constexpr int BR = 256;
  const int nqb = (a.N + BR - 1) / BR;
  const long long nblocks = (long long)a.B * a.Hq * nqb;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)nblocks), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_fwd_fp8_t<128, true>(a, stream) : launch_fwd_fp8_t<128, false>(a, stream);
  return causal ? launch_fwd_fp8_t<64, true>(a, stream) : launch_fwd_fp8_t<64, false>(a, stream);
}

}  // namespace fa
