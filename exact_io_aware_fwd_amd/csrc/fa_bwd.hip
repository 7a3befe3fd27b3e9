// Backward pass of exact attention for gfx950, by recomputation from the saved LSE.
//
// Method: "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section
// "Backward pass: recomputation instead of storage" (Figure 5): only O and the
// per-row log-sum-exp are kept from the forward; S_ij and P_ij are recomputed
// tile by tile, dV_j and dK_j accumulate over query blocks, and dQ_i accumulates
// over key blocks with atomic adds.  The page's dS omits the softmax-Jacobian
// term; the full gradient is used: dS = P * (dP - D) with D_i = sum_k dO_ik O_ik,
// and the softmax scale multiplies dQ and dK.
//
// Three kernels on the caller's stream:
//  1. row terms: D_i in fp32, and the fp32 dQ accumulator cleared;
//  2. main: one workgroup per (batch, K/V head, 128-key block).  Each of the 4
//     waves owns 32 keys and keeps dK^T, dV^T for them in registers across all
//     query heads of the group and all query blocks (from the diagonal when
//     causal).  Per 32-query step, with v_mfma_f32_32x32x16:
//        S  = Q K^T,  dP = dO V^T          (lane = key, rows = queries)
//        P  = exp2(S*scale*log2e - LSE*log2e),  dS = P * (dP - D)
//        dV^T += dO^T P,  dK^T += Q^T dS   (P, dS stay in registers as B operands;
//                                           Q^T and dO^T come from LDS through
//                                           ds_read_b64_tr_b16)
//        dS -> LDS, then each wave forms dQ for 32 of the d columns over all
//        128 keys and adds it to the fp32 accumulator with atomics;
//  3. dQ = scale * accumulator, rounded to the input dtype.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// ---- 1. D_i = sum_k dO_ik O_ik and dQ accumulator = 0 --------------------------------
template <class Tag, int D>
__global__ void __launch_bounds__(256) bwd_rowterm_kernel(const BwdArgs a, long long rows) {
  using E = Elt<Tag>;
  constexpr int TPR = D / 8;   // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o4 = *(const u32x4*)((const unsigned char*)a.o + (row * D + part * 8) * 2);
    const u32x4 g4 = *(const u32x4*)((const unsigned char*)a.dout + (row * D + part * 8) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += E::to_f32((uint16_t)(o4[i] & 0xffff)) * E::to_f32((uint16_t)(g4[i] & 0xffff));
      acc += E::to_f32((uint16_t)(o4[i] >> 16)) * E::to_f32((uint16_t)(g4[i] >> 16));
    }
    float* z = a.dqacc + row * D + part * 8;
    *(f32x4*)z = f32x4{0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(z + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && part == 0) a.dsum[row] = acc;
}

// ---- 2. main: dK, dV per key block; dQ by atomics --------------------------------------
template <class Tag, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) bwd_main_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  constexpr int NW = 4, NT = 256;
  constexpr int BKV = 32 * NW;     // keys per workgroup
  constexpr int BQ = 32;           // queries per step
  constexpr int ROWB = D * 2;
  constexpr int PK = ROWB + 16;    // K, V rows in LDS
  constexpr int PQ = ROWB + 32;    // Q, dO rows in LDS (also read transposed)
  constexpr int PS = BKV * 2 + 16; // dS rows [query][key]
  constexpr int KV_BYTES = BKV * PK;
  constexpr int QT_BYTES = BQ * PQ;
  constexpr int CH_ROW = D / 8;
  constexpr int QCH = BQ * CH_ROW;       // 16-byte chunks per Q (or dO) tile
  constexpr int QCPT = 2 * QCH / NT;     // per thread per step
  static_assert(QCPT * NT == 2 * QCH && QCH % NT == 0, "step load split");

  __shared__ __attribute__((aligned(16))) unsigned char Ks[KV_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char Vs[KV_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char Qs[2][QT_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char dOs[2][QT_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char dSs[BQ * PS];
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
  __shared__ __attribute__((aligned(16))) float dsums[2][BQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;
  const int G = a.Hq / a.Hkv;
  const int nkb = (N + BKV - 1) / BKV;
  const int ngroups = a.B * a.Hkv;
  const int jb = blockIdx.x / ngroups;          // key blocks nearest the start first (most work)
  const int grp = blockIdx.x - jb * ngroups;
  const int b = grp / a.Hkv, hkv = grp - b * a.Hkv;
  (void)nkb;

  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
  const int k0 = jb * BKV;
  const int kw = k0 + 32 * wave;     // first key of this wave
  const int mykey = kw + r32;        // the key this lane's scores belong to

  // K and V tiles for the whole workgroup (rows past the end are zero)
  {
    const unsigned char* Kg = (const unsigned char*)a.k + kvhead * ROWB;
    const unsigned char* Vg = (const unsigned char*)a.v + kvhead * ROWB;
    for (int ci = tid; ci < BKV * CH_ROW; ci += NT) {
      const int row = ci / CH_ROW, col = ci - (ci / CH_ROW) * CH_ROW;
      u32x4 kx = u32x4{0, 0, 0, 0}, vx = u32x4{0, 0, 0, 0};
      if (k0 + row < N) {
        kx = *(const u32x4*)(Kg + (size_t)(k0 + row) * ROWB + col * 16);
        vx = *(const u32x4*)(Vg + (size_t)(k0 + row) * ROWB + col * 16);
      }
      *(u32x4*)(Ks + row * PK + col * 16) = kx;
      *(u32x4*)(Vs + row * PK + col * 16) = vx;
    }
  }

  const int iq0 = CAUSAL ? k0 / BQ : 0;
  const int nqb = (N + BQ - 1) / BQ;
  const int per_head = nqb - iq0;
  const int nsteps = G * per_head;

  u32x4 stage[QCPT];
  float stage_l = 0.f;
  auto gload = [&](int step) {
    const int g = step / per_head;
    const int qb = (iq0 + (step - g * per_head)) * BQ;
    const size_t qhead = (size_t)(b * a.Hq + hkv * G + g) * (size_t)N;
    const bool full = qb + BQ <= N;
#pragma unroll
    for (int c = 0; c < QCPT; ++c) {
      const int ci = tid + c * NT;
      const int tens = (c * NT) / QCH;   // 0 = Q, 1 = dO
      const int w = ci - tens * QCH;
      const int row = w / CH_ROW, col = w - (w / CH_ROW) * CH_ROW;
      const unsigned char* src = (const unsigned char*)(tens == 0 ? a.q : a.dout) +
                                 ((qhead + qb + row) * ROWB) + col * 16;
      stage[c] = (full || qb + row < N) ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
    }
    if (tid < 2 * BQ) {
      const int r = tid & (BQ - 1);
      if (qb + r < N)
        stage_l = (tid < BQ) ? a.lse[qhead + qb + r] * kLog2e : a.dsum[qhead + qb + r];
      else
        stage_l = 0.f;
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int c = 0; c < QCPT; ++c) {
      const int ci = tid + c * NT;
      const int tens = (c * NT) / QCH;
      const int w = ci - tens * QCH;
      const int row = w / CH_ROW, col = w - (w / CH_ROW) * CH_ROW;
      unsigned char* dst = (tens == 0 ? Qs[buf] : dOs[buf]) + row * PQ + col * 16;
      *(u32x4*)dst = stage[c];
    }
    if (tid < 2 * BQ) {
      if (tid < BQ) lse2s[buf][tid] = stage_l;
      else dsums[buf][tid - BQ] = stage_l;
    }
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      dk[e][v] = 0.f;
      dv[e][v] = 0.f;
    }

  const float c2 = a.scale_log2;
  const int rowoff = r32 * PQ + 16 * hh;                       // Q/dO row reads
  const int keyoff = (32 * wave + r32) * PK + 16 * hh;         // K/V row reads
  const int troff = (4 * hh + ((lane & 15) >> 2)) * PQ + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  const int ktroff = (8 * hh + ((lane & 15) >> 2)) * PK +
                     (32 * wave + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;  // K read transposed for dQ

  if (nsteps > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const int g = step / per_head;
    const int qb = (iq0 + (step - g * per_head)) * BQ;
    const size_t qhead = (size_t)(b * a.Hq + hkv * G + g) * (size_t)N;
    if (step + 1 < nsteps) gload(step + 1);

    const unsigned char* Qb = Qs[buf];
    const unsigned char* dOb = dOs[buf];
    // S = Q K^T and dP = dO V^T for (32 queries) x (this wave's 32 keys)
    f32x16 s, dp;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s[v] = 0.f;
      dp[v] = 0.f;
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      s = E::mma(*(const u32x4*)(Qb + rowoff + 32 * st), *(const u32x4*)(Ks + keyoff + 32 * st), s);
      dp = E::mma(*(const u32x4*)(dOb + rowoff + 32 * st), *(const u32x4*)(Vs + keyoff + 32 * st), dp);
    }
    // P and dS; lane holds key `mykey`, rows q = 8*(v/4) + 4*hh + v%4
    float lse2[16], dsv[16];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const f32x4 l4 = *(const f32x4*)&lse2s[buf][8 * a4 + 4 * hh];
      const f32x4 d4 = *(const f32x4*)&dsums[buf][8 * a4 + 4 * hh];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lse2[4 * a4 + i] = l4[i];
        dsv[4 * a4 + i] = d4[i];
      }
    }
    const bool need_mask = (qb + BQ > N) || (k0 + BKV > N) || (CAUSAL && kw + 31 > qb);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float p = fast_exp2(fmaf(s[v], c2, -lse2[v]));
      if (need_mask) {
        const int q = qb + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (q >= N || mykey >= N || (CAUSAL && mykey > q)) p = 0.f;
      }
      s[v] = p;
      dp[v] = p * (dp[v] - dsv[v]);
    }
    u32x4 pf[2], sf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int v0 = 8 * t;
      pf[t] = u32x4{E::pack(s[v0 + 0], s[v0 + 1]), E::pack(s[v0 + 2], s[v0 + 3]),
                    E::pack(s[v0 + 4], s[v0 + 5]), E::pack(s[v0 + 6], s[v0 + 7])};
      sf[t] = u32x4{E::pack(dp[v0 + 0], dp[v0 + 1]), E::pack(dp[v0 + 2], dp[v0 + 3]),
                    E::pack(dp[v0 + 4], dp[v0 + 5]), E::pack(dp[v0 + 6], dp[v0 + 7])};
    }
    // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 ado = cat(lds_read_tr(dOb + troff + 16 * t * PQ + 64 * e),
                              lds_read_tr(dOb + troff + (16 * t + 8) * PQ + 64 * e));
        dv[e] = E::mma(ado, pf[t], dv[e]);
        const u32x4 aq = cat(lds_read_tr(Qb + troff + 16 * t * PQ + 64 * e),
                             lds_read_tr(Qb + troff + (16 * t + 8) * PQ + 64 * e));
        dk[e] = E::mma(aq, sf[t], dk[e]);
      }
    // dS (rounded to the input dtype, as used above) -> LDS as [query][key]
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int qr = 8 * (v >> 2) + 4 * hh + (v & 3);
      const uint32_t pk = E::pack(dp[v], 0.f);
      *(uint16_t*)(dSs + qr * PS + (32 * wave + r32) * 2) = (uint16_t)(pk & 0xffff);
    }
    __syncthreads();
    // dQ[q][32*wave + r32] over the 128 keys of the block (d = 64: waves 2, 3 idle here)
    if (32 * wave < D) {
      f32x16 dq;
#pragma unroll
      for (int v = 0; v < 16; ++v) dq[v] = 0.f;
#pragma unroll
      for (int st = 0; st < BKV / 16; ++st) {
        const u32x4 ads = *(const u32x4*)(dSs + r32 * PS + (16 * st + 8 * hh) * 2);
        const u32x4 bk = cat(lds_read_tr(Ks + ktroff + 16 * st * PK), lds_read_tr(Ks + ktroff + (16 * st + 4) * PK));
        dq = E::mma(ads, bk, dq);
      }
      float* dqa = a.dqacc + (qhead + qb) * D + 32 * wave + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int qr = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (qb + qr < N) atomicAdd(dqa + (size_t)qr * D, dq[v]);
      }
    }
    if (step + 1 < nsteps) swrite(buf ^ 1);
    __syncthreads();
  }

  // dK = scale * dK^T^T, dV = dV^T^T, rounded to the input dtype
  if (mykey < N) {
    unsigned char* dKg = (unsigned char*)a.dk + (kvhead + mykey) * ROWB;
    unsigned char* dVg = (unsigned char*)a.dv + (kvhead + mykey) * ROWB;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * e + 8 * g4 + 4 * hh;
        const u32x2 wk = {E::pack(dk[e][4 * g4 + 0] * a.scale, dk[e][4 * g4 + 1] * a.scale),
                          E::pack(dk[e][4 * g4 + 2] * a.scale, dk[e][4 * g4 + 3] * a.scale)};
        const u32x2 wv = {E::pack(dv[e][4 * g4 + 0], dv[e][4 * g4 + 1]),
                          E::pack(dv[e][4 * g4 + 2], dv[e][4 * g4 + 3])};
        *(u32x2*)(dKg + d0 * 2) = wk;
        *(u32x2*)(dVg + d0 * 2) = wv;
      }
  }
}

// ---- 3. dQ = scale * accumulator ---------------------------------------------------------
template <class Tag>
__global__ void __launch_bounds__(256) bwd_dq_kernel(const BwdArgs a, long long n8) {
  using E = Elt<Tag>;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x0 = *(const f32x4*)(a.dqacc + i * 8);
  const f32x4 x1 = *(const f32x4*)(a.dqacc + i * 8 + 4);
  const float s = a.scale;
  const u32x4 w = {E::pack(x0[0] * s, x0[1] * s), E::pack(x0[2] * s, x0[3] * s),
                   E::pack(x1[0] * s, x1[1] * s), E::pack(x1[2] * s, x1[3] * s)};
  *(u32x4*)((unsigned char*)a.dq + i * 16) = w;
}

template <class Tag, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.N;
  if (rows <= 0) return hipSuccess;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_rowterm_kernel<Tag, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, a, rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long nkb = (a.N + 127) / 128;
  hipLaunchKernelGGL((bwd_main_kernel<Tag, D, CAUSAL>), dim3((unsigned)(nkb * a.B * a.Hkv)), dim3(256), 0,
                     stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL((bwd_dq_kernel<Tag>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, a, n8);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16, bool causal, hipStream_t stream) {
#define FA_BWD_CASE(TAG, D) \
  return causal ? launch_bwd_t<TAG, D, true>(a, stream) : launch_bwd_t<TAG, D, false>(a, stream)
  if (bf16) {
    if (d == 128) FA_BWD_CASE(bf16_tag, 128);
    FA_BWD_CASE(bf16_tag, 64);
  } else {
    if (d == 128) FA_BWD_CASE(f16_tag, 128);
    FA_BWD_CASE(f16_tag, 64);
  }
#undef FA_BWD_CASE
}

}  // namespace fa
