// Forward pass of exact attention for gfx950: tiled, online softmax, O and LSE only.
//
// Method: "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section
// "FlashAttention-1: tiling plus online softmax" (Figures 3 and 4): Q row blocks
// outer, K/V column blocks inner, running max m, running sum l and unnormalised
// output kept on chip, one division at the end; causal tiles above the diagonal
// are skipped.  Work split as in the section "FlashAttention-2: better work
// partitioning" (Figure 6): one workgroup per (batch, head, query block), so no
// atomics and a bitwise-deterministic result.
//
// gfx950 design.
//  * A workgroup owns BR = 32*NW query rows; wave w owns rows [32w, 32w+32).
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: every
//    lane then holds the scores of ONE query (lane % 32) for 32 keys, so the row
//    max and row sum are in-lane plus one permlane32 swap, and the probabilities
//    are already in the B-operand layout of O^T += V^T P^T (no LDS round trip).
//    The key order inside each 16-key MFMA step is permuted consistently on both
//    operands, which the sum over keys does not see.
//  * Q stays in VGPRs for the whole key loop; K and V tiles (BC = 64 keys) are
//    double-buffered in LDS, prefetched from HBM into VGPRs one tile ahead.
//  * V stays row-major in LDS; ds_read_b64_tr_b16 delivers it transposed as the
//    A operand.
//  * Scores are kept in log2 units: p = exp2(s * scale*log2e - m * scale*log2e).
//  * Causal: a workgroup stops at the last tile its rows can see; inside the
//    diagonal band a wave skips tiles entirely above its rows and masks only
//    tiles that cross its diagonal (or the sequence end).
//  * Block ids are remapped so that all query blocks sharing a K/V head run on
//    one XCD (block ids are dealt round-robin over the 8 XCDs) and the longest
//    causal blocks start first.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// Block id -> (batch, query head, query block).  Blocks are dealt round-robin to
// the 8 XCDs; when the number of (batch, kv-head) groups is a multiple of 8,
// XCD x serves groups x, x+8, ... so their K/V stay in that XCD's L2.  Within an
// XCD, slots run over query blocks from the last (longest when causal) down.
__device__ __forceinline__ void map_fwd_block(int nqb, int B, int Hq, int Hkv, int& b, int& hq,
                                              int& iq) {
  const int G = Hq / Hkv;
  const int ngroups = B * Hkv;
  const int bid = blockIdx.x;
  int grp, gq, iq_rev;
  if ((ngroups & 7) == 0) {
    const int x = bid & 7, s = bid >> 3;
    const int per = (ngroups >> 3) * G;  // blocks per query-block index on one XCD
    iq_rev = s / per;
    const int rest = s - iq_rev * per;
    grp = x + 8 * (rest / G);
    gq = rest - (rest / G) * G;
  } else {
    const int per = ngroups * G;
    iq_rev = bid / per;
    const int rest = bid - iq_rev * per;
    grp = rest / G;
    gq = rest - grp * G;
  }
  iq = nqb - 1 - iq_rev;
  b = grp / Hkv;
  hq = (grp - b * Hkv) * G + gq;
}

template <class Tag, int D, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64) fwd_kernel(const FwdArgs a) {
  using E = Elt<Tag>;
  constexpr int BR = 32 * NW;          // query rows per workgroup
  constexpr int BC = 64;               // keys per tile
  constexpr int NT = NW * 64;          // threads
  constexpr int ROWB = D * 2;          // bytes of one K/V/Q/O row
  constexpr int PK = ROWB + 16;        // LDS pitch of K rows (row-contiguous 16-byte reads)
  constexpr int PV = ROWB + 32;        // LDS pitch of V rows (transposing 8-byte reads)
  constexpr int KT = BC * PK;
  constexpr int STAGE = KT + BC * PV;
  constexpr int CH_ROW = D / 8;        // 16-byte chunks per row
  constexpr int CH_T = BC * CH_ROW;    // chunks per K (or V) tile
  constexpr int CPT = 2 * CH_T / NT;   // chunks each thread moves per tile
  static_assert(CPT * NT == 2 * CH_T && CH_T % NT == 0, "tile load split");

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;

  int b, hq, iq;
  map_fwd_block((N + BR - 1) / BR, a.B, a.Hq, a.Hkv, b, hq, iq);
  const int hkv = hq / (a.Hq / a.Hkv);
  const size_t qhead = (size_t)(b * a.Hq + hq) * (size_t)N;
  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
  const unsigned char* Qg = (const unsigned char*)a.q + qhead * ROWB;
  const unsigned char* Kg = (const unsigned char*)a.k + kvhead * ROWB;
  const unsigned char* Vg = (const unsigned char*)a.v + kvhead * ROWB;

  const int q0 = iq * BR;
  const int qw = q0 + wave * 32;   // first row of this wave
  const int myq = qw + r32;        // the query this lane's scores belong to

  // Q^T as the B operand: lane holds Q[myq][16s + 8hh .. +7]
  u32x4 qf[D / 16];
  if (myq < N) {
    const unsigned char* qp = Qg + (size_t)myq * ROWB + 16 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *(const u32x4*)(qp + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = u32x4{0, 0, 0, 0};
  }

  const int nkv = (N + BC - 1) / BC;
  int ntile = nkv;
  if (CAUSAL) ntile = min(nkv, (min(q0 + BR, N) - 1) / BC + 1);

  u32x4 stage[CPT];
  auto gload = [&](int j) {
    const int kbase = j * BC;
    const bool full = kbase + BC <= N;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * NT;
      const int tens = (c * NT) / CH_T;  // compile-time: 0 = K, 1 = V
      const int w = ci - tens * CH_T;
      const int row = w / CH_ROW, col = w - (w / CH_ROW) * CH_ROW;
      const unsigned char* src = (tens == 0 ? Kg : Vg) + (size_t)(kbase + row) * ROWB + col * 16;
      if (full || kbase + row < N)
        stage[c] = *(const u32x4*)src;
      else
        stage[c] = u32x4{0, 0, 0, 0};   // rows past the end: zero, so 0 * V stays finite
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ci = tid + c * NT;
      const int tens = (c * NT) / CH_T;
      const int w = ci - tens * CH_T;
      const int row = w / CH_ROW, col = w - (w / CH_ROW) * CH_ROW;
      unsigned char* dst = smem + buf * STAGE + (tens == 0 ? row * PK : KT + row * PV) + col * 16;
      *(u32x4*)dst = stage[c];
    }
  };

  const float c2 = a.scale_log2;
  float m_run = -INFINITY;   // running max of the raw scores of query myq
  float l_run = 0.f;         // running sum over this lane's half of the keys
  f32x16 o[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[e][v] = 0.f;

  // per-lane LDS offsets
  const int koff = r32 * PK + 16 * hh;
  const int voff = (4 * hh + ((lane & 15) >> 2)) * PV + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  gload(0);
  swrite(0);
  __syncthreads();

  for (int j = 0; j < ntile; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntile) gload(j + 1);
    const unsigned char* Ks = smem + buf * STAGE;
    const unsigned char* Vs = Ks + KT;
    const int k0 = j * BC;
    if (!CAUSAL || k0 <= qw + 31) {
      // S^T = K Q^T, two 32-key halves
      f32x16 s[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[c][v] = 0.f;
        const unsigned char* kp = Ks + 32 * c * PK + koff;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) s[c] = E::mma(*(const u32x4*)(kp + 32 * st), qf[st], s[c]);
      }
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + 32 * c + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (key >= N || (CAUSAL && key > myq)) s[c][v] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[c][v]);
      mx = half_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float mref = (m_new == -INFINITY) ? 0.f : m_new * c2;
      const float alpha = fast_exp2(m_run * c2 - mref);
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(fmaf(s[c][v], c2, -mref));
          s[c][v] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[e][v] *= alpha;
      // P^T as the B operand: step t covers keys [16t, 16t+16)
      u32x4 pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = t >> 1, v0 = 8 * (t & 1);
        pf[t] = u32x4{E::pack(s[c][v0 + 0], s[c][v0 + 1]), E::pack(s[c][v0 + 2], s[c][v0 + 3]),
                      E::pack(s[c][v0 + 4], s[c][v0 + 5]), E::pack(s[c][v0 + 6], s[c][v0 + 7])};
      }
      // O^T += V^T P^T
      const unsigned char* vp = Vs + voff;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4 af = cat(lds_read_tr(vp + 16 * t * PV + 64 * e), lds_read_tr(vp + (16 * t + 8) * PV + 64 * e));
          o[e] = E::mma(af, pf[t], o[e]);
        }
    }
    if (j + 1 < ntile) swrite(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = O^T / l, LSE = ln(2) * (m*scale*log2e + log2 l)
  const float l_tot = half_sum(l_run);
  if (myq < N) {
    const float inv = 1.f / l_tot;
    unsigned char* Og = (unsigned char*)a.o + (qhead + myq) * ROWB;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * e + 8 * g + 4 * hh;
        const u32x2 w = {E::pack(o[e][4 * g + 0] * inv, o[e][4 * g + 1] * inv),
                         E::pack(o[e][4 * g + 2] * inv, o[e][4 * g + 3] * inv)};
        *(u32x2*)(Og + d0 * 2) = w;
      }
    if (hh == 0) {
      const float mref = m_run * c2;
      a.lse[qhead + myq] = (mref + log2f(l_tot)) * kLn2;
    }
  }
}

template <class Tag, int D, int NW, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const int nqb = (a.N + BR - 1) / BR;
  const long long nblocks = (long long)a.B * a.Hq * nqb;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<Tag, D, NW, CAUSAL>), dim3((unsigned)nblocks), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16, bool causal, hipStream_t stream) {
  constexpr int NW = 8;
#define FA_FWD_CASE(TAG, D)                                                       \
  return causal ? launch_fwd_t<TAG, D, NW, true>(a, stream) : launch_fwd_t<TAG, D, NW, false>(a, stream)
  if (bf16) {
    if (d == 128) FA_FWD_CASE(bf16_tag, 128);
    FA_FWD_CASE(bf16_tag, 64);
  } else {
    if (d == 128) FA_FWD_CASE(f16_tag, 128);
    FA_FWD_CASE(f16_tag, 64);
  }
#undef FA_FWD_CASE
}

}  // namespace fa
