// Backward pass of exact attention for gfx950, by recomputation from the saved LSE.
//
// Method: "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section
// "Backward pass: recomputation instead of storage" (Figure 5): only O and the
// per-row log-sum-exp are kept from the forward; S_ij and P_ij are recomputed
// tile by tile.  The page's dS omits the softmax-Jacobian term; the full gradient
// is used: dS = P * (dP - D) with D_i = sum_k dO_ik O_ik, and the softmax scale
// multiplies dQ and dK.
//
// The page's kernel accumulates dQ across key blocks with atomic adds.  On a
// multi-XCD gfx950 every device-scope float atomic leaves the XCD's L2 for the
// memory fabric (measured: ~9 GB of fabric writes per backward at N=8192, d=128),
// so this backward instead splits the work into two passes that each own their
// output, as the same section's deterministic option does: it recomputes S and dP
// once more, needs no atomics and no fp32 dQ buffer, and is bitwise reproducible.
//
//  1. row terms: D_i = sum_k dO_ik O_ik in fp32;
//  2. dQ pass: one workgroup per (batch, head, 32*NW-query block), the forward's
//     structure: S^T = K Q^T and dP^T = V dO^T with Q, dO in VGPRs and K, V tiles
//     streamed through LDS; P = exp2(S*scale*log2e - LSE*log2e),
//     dS = P * (dP - D) in registers, dQ^T += K^T dS^T (K read transposed);
//  3. dK/dV pass: one workgroup per (batch, K/V head, 128-key block); each of the
//     4 waves owns 32 keys and keeps dK^T, dV^T for them in registers across all
//     query heads of the group and all query blocks (from the diagonal when
//     causal).  Per 32-query step: S = Q K^T, dP = dO V^T (lane = key),
//     dV^T += dO^T P, dK^T += Q^T dS (Q^T, dO^T read transposed from LDS).
#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// ---- 1. D_i = sum_k dO_ik O_ik --------------------------------------------------------
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
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && part == 0) a.dsum[row] = acc;
}

// ---- 3. dK, dV per key block ---------------------------------------------------------
template <class Tag, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  constexpr int NW = 4, NT = 256;
  constexpr int BKV = 32 * NW;     // keys per workgroup
  constexpr int BQ = 32;           // queries per step
  constexpr int ROWB = D * 2;
  constexpr int PK = ROWB + 16;    // K, V rows in LDS
  constexpr int PQ = ROWB + 32;    // Q, dO rows in LDS (also read transposed)
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

  if (nsteps > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const int g = step / per_head;
    const int qb = (iq0 + (step - g * per_head)) * BQ;
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

// ---- 2. dQ per query block -------------------------------------------------------------
template <class Tag, int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(NW * 64) bwd_dq_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  constexpr int BR = 32 * NW;           // query rows per workgroup
  constexpr int BC = 64;                // keys per tile
  constexpr int ROWB = D * 2;
  constexpr int PK = ROWB + 64;         // K rows: read as rows (S^T) and transposed (dQ^T)
  constexpr int PV = ROWB + 16;         // V rows: read as rows (dP^T)
  using Tiles = TilePair<ROWB, PK, PV, NW>;
  constexpr int KBYTES = Tiles::ABYTES;
  constexpr int SLOT = Tiles::SLOT;
  constexpr int IPW = Tiles::IPW;
  constexpr int NE = D / 32;            // 32-row blocks of dQ^T
  constexpr int NS = D / 16;            // k-steps of S^T and dP^T

  __shared__ __attribute__((aligned(1024))) unsigned char lds[3 * SLOT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;

  int b, hq, iq;
  map_q_block((N + BR - 1) / BR, a.B, a.Hq, a.Hkv, b, hq, iq);
  const int hkv = hq / (a.Hq / a.Hkv);
  const size_t qhead = (size_t)(b * a.Hq + hq) * (size_t)N;
  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
  const unsigned char* Kg = (const unsigned char*)a.k + kvhead * ROWB;
  const unsigned char* Vg = (const unsigned char*)a.v + kvhead * ROWB;

  const int q0 = iq * BR;
  const int qw = q0 + wave * 32;
  const int myq = qw + r32;            // the query this lane's scores belong to

  // Q^T and dO^T as B operands: lane holds row myq, elements 16s + 8hh .. +7
  u32x4 qf[NS], df[NS];
  float lse2 = 0.f, dsv = 0.f;
  if (myq < N) {
    const unsigned char* qp = (const unsigned char*)a.q + (qhead + myq) * ROWB + 16 * hh;
    const unsigned char* gp = (const unsigned char*)a.dout + (qhead + myq) * ROWB + 16 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = *(const u32x4*)(qp + 32 * s);
      df[s] = *(const u32x4*)(gp + 32 * s);
    }
    lse2 = a.lse[qhead + myq] * kLog2e;
    dsv = a.dsum[qhead + myq];
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = df[s] = u32x4{0, 0, 0, 0};
  }

  const int nkv = (N + BC - 1) / BC;
  const int ntile = CAUSAL ? min(nkv, (min(q0 + BR, N) - 1) / BC + 1) : nkv;

  int doff[IPW];
  Tiles::offsets(wave, lane, doff);
  auto dma = [&](int t) { Tiles::load(Kg, Vg, N, t, wave, doff, lds + (t % 3) * SLOT); };

  // per-lane LDS offsets: K and V rows (A operands of S^T, dP^T), K transposed (A of dQ^T)
  const int ka = r32 * PK + 16 * hh;
  const int va = KBYTES + r32 * PV + 16 * hh;
  const int kt = (4 * hh + ((lane & 15) >> 2)) * PK + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  const float c2 = a.scale_log2;
  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = zero16();

  // unit u = 32 keys = half (u & 1) of tile u >> 1
  auto ubase = [&](int u, int half_pitch) {
    int r = ((u >> 1) % 3) * SLOT + (u & 1) * 32 * half_pitch;
    opaque(r);
    return r;
  };
  auto krow = [&](int kb, int st) { return *(const u32x4*)(lds + kb + ka + 32 * st); };
  auto vrow = [&](int kb, int st) { return *(const u32x4*)(lds + kb + va + 32 * st); };
  auto ktr = [&](int kb, int h, int e) {
    return cat(lds_read_tr(lds + kb + kt + 16 * h * PK + 64 * e), lds_read_tr(lds + kb + kt + (16 * h + 8) * PK + 64 * e));
  };
  // dS of one unit from its S^T and dP^T, packed as the B operand of two 16-key steps
  auto dsfrom = [&](f32x16& s, const f32x16& dp, int lo, int hi) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (v >= lo && v < hi) {
        const float p = fast_exp2(fmaf(s[v], c2, -lse2));
        s[v] = p * (dp[v] - dsv);
        keep(s[v]);
      }
  };
  auto pack = [&](const f32x16& s, int h) {
    return u32x4{E::pack(s[8 * h + 0], s[8 * h + 1]), E::pack(s[8 * h + 2], s[8 * h + 3]),
                 E::pack(s[8 * h + 4], s[8 * h + 5]), E::pack(s[8 * h + 6], s[8 * h + 7])};
  };

  const int ulast = (CAUSAL ? min(qw + 31, N - 1) : N - 1) / 32;

  // Unit u < ulast: products of unit u+1 interleaved with the elementwise dS of unit u,
  // then dQ^T += K_u^T dS_u^T.
  auto step_main = [&](int u, f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn) {
    const int kn = ubase(u + 1, PK), vn = ubase(u + 1, PV), kc = ubase(u, PK);
    u32x4 kf = krow(kn, 0), vf = vrow(vn, 0);
    u32x4 pf[2];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k == 0) {
        sn = zero16();
        dpn = zero16();
      }
      sn = E::mma(kf, qf[k], sn);
      dpn = E::mma(vf, df[k], dpn);
      if (k + 1 < NS) {
        kf = krow(kn, k + 1);
        vf = vrow(vn, k + 1);
      }
      dsfrom(sc, dpc, (16 * k) / NS, (16 * (k + 1)) / NS);
      if (k == NS - 1) {
        pf[0] = pack(sc, 0);
        pf[1] = pack(sc, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 tf = ktr(kc, 0, 0);
#pragma unroll
    for (int k = 0; k < 2 * NE; ++k) {
      const int h = k / NE, e = k % NE;
      const u32x4 cur = tf;
      if (k + 1 < 2 * NE) tf = ktr(kc, (k + 1) / NE, (k + 1) % NE);
      acc[e] = E::mma(cur, pf[h], acc[e]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The wave's last unit: diagonal (causal) and/or sequence tail.
  auto step_last = [&](int u, f32x16& sc, const f32x16& dpc) {
    const int k0 = u * 32;
    int lim = N - k0 - 4 * hh;
    if (CAUSAL) lim = min(lim, myq - k0 - 4 * hh + 1);
    dsfrom(sc, dpc, 0, 16);
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (8 * (v >> 2) + (v & 3) >= lim) sc[v] = 0.f;
    const u32x4 pf[2] = {pack(sc, 0), pack(sc, 1)};
    const int kc = ubase(u, PK);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] = E::mma(ktr(kc, h, e), pf[h], acc[e]);
  };

  auto step = [&](int u, f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn) {
    if (u < ulast) step_main(u, sc, dpc, sn, dpn);
    else if (u == ulast) step_last(u, sc, dpc);
  };

  dma(0);
  if (ntile > 1) dma(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x16 sa, pa, sb, pb;
  {
    const int k0 = ubase(0, PK), v0 = ubase(0, PV);
    sa = zero16();
    pa = zero16();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      sa = E::mma(krow(k0, st), qf[st], sa);
      pa = E::mma(vrow(v0, st), df[st], pa);
    }
  }
  const int ulast0 = (CAUSAL ? min(q0 + 31, N - 1) : N - 1) / 32;
  const int J1 = min(ntile, ulast0 / 2);
  auto tile_start = [&](int j) {
    if (j > 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (j + 2 < ntile) dma(j + 2);
  };
  for (int j = 0; j < J1; ++j) {
    tile_start(j);
    step_main(2 * j, sa, pa, sb, pb);
    step_main(2 * j + 1, sb, pb, sa, pa);
  }
  for (int j = J1; j < ntile; ++j) {
    tile_start(j);
    step(2 * j, sa, pa, sb, pb);
    step(2 * j + 1, sb, pb, sa, pa);
  }

  // dQ = scale * (dQ^T)^T, rounded to the input dtype
  if (myq < N) {
    unsigned char* Og = (unsigned char*)a.dq + (qhead + myq) * ROWB;
    const float sc = a.scale;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * e + 8 * g + 4 * hh;
        const u32x2 w = {E::pack(acc[e][4 * g + 0] * sc, acc[e][4 * g + 1] * sc),
                         E::pack(acc[e][4 * g + 2] * sc, acc[e][4 * g + 3] * sc)};
        *(u32x2*)(Og + d0 * 2) = w;
      }
  }
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
  // d = 128: Q, dO, the dQ accumulator and two units of S, dP need more than the 256
  // registers a wave has at two waves per SIMD, so that case runs 4 waves (1 per SIMD).
  constexpr int NWQ = D == 128 ? 4 : 8;
  const long long nqb = (a.N + 32 * NWQ - 1) / (32 * NWQ);
  hipLaunchKernelGGL((bwd_dq_kernel<Tag, D, CAUSAL, NWQ>), dim3((unsigned)(nqb * a.B * a.Hq)), dim3(NWQ * 64), 0,
                     stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long nkb = (a.N + 127) / 128;
  hipLaunchKernelGGL((bwd_dkdv_kernel<Tag, D, CAUSAL>), dim3((unsigned)(nkb * a.B * a.Hkv)), dim3(256), 0,
                     stream, a);
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
