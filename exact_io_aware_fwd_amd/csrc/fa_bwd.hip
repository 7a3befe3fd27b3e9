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
//  1. row terms: LSE_i * log2(e) and D_i = sum_k dO_ik O_ik in fp32, as pairs;
//  2. dQ pass: one workgroup per (batch, head, 32*NW-query block), the forward's
//     structure: S^T = K Q^T and dP^T = V dO^T with Q, dO in VGPRs and K (XOR-
//     swizzled: read by rows and transposed), V tiles streamed through LDS;
//     P = exp2(S*scale*log2e - LSE*log2e),
//     dS = P * (dP - D) in registers, dQ^T += K^T dS^T (K read transposed);
//  3. dK/dV pass: one workgroup per (batch, K/V head, 128-key block); each of the
//     4 waves owns 32 keys, holds their K and V in VGPRs and dK^T, dV^T in
//     accumulators across all query heads of the group and all query blocks (from
//     the diagonal when causal; query blocks descending, heads inner, so that
//     concurrent workgroups share Q/dO tiles in L2).  Q, dO and the row terms of each 32-query step go
//     HBM -> LDS directly (three slots, two steps in flight).  Per step:
//     S = Q K^T, dP = dO V^T (lane = key), dV^T += dO^T P, dK^T += Q^T dS (Q^T,
//     dO^T read transposed from LDS); the products of step n+1 are interleaved
//     with the elementwise work of step n.
#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// ---- 1. row terms: (LSE_i * log2 e, D_i = sum_k dO_ik O_ik) per query row ------------
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
  if (row < rows && part == 0) {
    a.rowterm[2 * row] = a.lse[row] * kLog2e;
    a.rowterm[2 * row + 1] = acc;
  }
}

// ---- 3. dK, dV per key block ---------------------------------------------------------
// Q rows, dO rows (TB bytes each, 16-byte chunks XOR-swizzled by soff) and the
// (LSE*log2e, D) row pairs of one query block into an LDS slot, straight from HBM.
// `rows` rows remain from the block's first row on; rows past them arrive as zeros.
// (A free function: the host pass of the compiler mishandles these builtins inside a
// capturing lambda.)
template <int ROWB, int TI, int LI, int NW, int TB>
__device__ __forceinline__ void dkdv_load_step(const BwdArgs& a, size_t qrow, int rows, int wave, int lane,
                                               const int* soff, unsigned char* slot) {
  const int bytes = rows * ROWB;
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const unsigned char*)a.q + qrow * ROWB), (short)0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const unsigned char*)a.dout + qrow * ROWB), (short)0, bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < LI; ++i) {
    const int nn = wave + NW * i;
    if (nn < TI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lvoid*)(slot + nn * 1024), 16, soff[i], 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lvoid*)(slot + nn * 1024), 16, soff[i], 0, 0, 0);
  }
  if (wave == 0) {
    const __amdgpu_buffer_rsrc_t rr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.rowterm + 2 * qrow), (short)0, rows * 8, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lvoid*)(slot + 2 * TB), 4, lane * 4, 0, 0, 0);
  }
}

template <class Tag, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  constexpr int NW = 4;
  constexpr int BKV = 32 * NW;        // keys per workgroup; wave w owns keys 32w .. 32w+31
  constexpr int BQ = 32;              // queries per step
  constexpr int ROWB = D * 2;
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int NS = D / 16;          // k-steps of S and dP
  constexpr int NE = D / 32;          // 32-row blocks of dK^T, dV^T
  constexpr int TB = BQ * ROWB;       // bytes of one Q (or dO) tile
  constexpr int TI = TB / 1024;       // wave-wide 16-byte-per-lane loads per tile
  constexpr int RPI = 1024 / ROWB;    // rows per such load
  constexpr int LI = (2 * TI + NW - 1) / NW;
  constexpr int SLOT = 2 * TB + BQ * 8;   // Q tile, dO tile, (LSE*log2e, D) pairs
  static_assert(2 * TI % NW == 0, "tile loads split evenly");

  __shared__ __attribute__((aligned(1024))) unsigned char lds[3 * SLOT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;
  const int G = a.Hq / a.Hkv;

  // block -> (key block, batch, kv head): groups x, x+8, ... on XCD x (their Q/dO stay in
  // one L2), key blocks nearest the start (the most causal work) first
  const int ngroups = a.B * a.Hkv;
  int jb, grp;
  if ((ngroups & 7) == 0) {
    const int x = blockIdx.x & 7, sidx = blockIdx.x >> 3, per = ngroups >> 3;
    jb = sidx / per;
    grp = x + 8 * (sidx - jb * per);
  } else {
    jb = blockIdx.x / ngroups;
    grp = blockIdx.x - jb * ngroups;
  }
  const int b = grp / a.Hkv, hkv = grp - b * a.Hkv;
  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
  const int k0 = jb * BKV;
  const int kw = k0 + 32 * wave;      // first key of this wave
  const int mykey = kw + r32;         // the key this lane's scores belong to

  // K^T and V^T as B operands: lane holds row mykey, elements 16s + 8hh .. +7
  u32x4 kf[NS], vf[NS];
  if (mykey < N) {
    const unsigned char* kp = (const unsigned char*)a.k + (kvhead + mykey) * ROWB + 16 * hh;
    const unsigned char* vp = (const unsigned char*)a.v + (kvhead + mykey) * ROWB + 16 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = *(const u32x4*)(kp + 32 * s);
      vf[s] = *(const u32x4*)(vp + 32 * s);
    }
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = vf[s] = u32x4{0, 0, 0, 0};
  }

  const int iq0 = CAUSAL ? k0 / BQ : 0;
  const int nqb = (N + BQ - 1) / BQ;
  const int per_head = nqb - iq0;
  const int nsteps = G * per_head;

  // ---- HBM -> LDS: step n into slot n % 3.  Tile load nn = wave + NW*i covers slot bytes
  // [1024nn, 1024nn+1024) (Q tile, then dO tile); lane's 16 bytes come from byte soff[i]
  // of the tile's rows (chunks XOR-swizzled).  Rows past N arrive as zeros.
  int soff[LI];
#pragma unroll
  for (int i = 0; i < LI; ++i) {
    const int nn = wave + NW * i;
    const int row = (nn % TI) * RPI + lane / CH;
    soff[i] = row * ROWB + (((lane % CH) ^ swz<CH>(row)) << 4);
  }
  // step n: query block nqb-1 - n/G (descending, so that the workgroups of a group walk
  // the same Q/dO tiles at the same time), query head hkv*G + n%G
  auto dma = [&](int n) __attribute__((always_inline)) {
    const int g = n % G;
    const int qb = (nqb - 1 - n / G) * BQ;
    const size_t qrow = (size_t)(b * a.Hq + hkv * G + g) * (size_t)N + qb;
    dkdv_load_step<ROWB, TI, LI, NW, TB>(a, qrow, N - qb, wave, lane, soff, lds + (n % 3) * SLOT);
  };

  // ---- per-lane LDS addresses (swizzled tiles) ----
  using SO = SwzOffsets<ROWB>;
  int rowa[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) rowa[st] = SO::rows_a0(lane) ^ (st << 5);
  int tra[2 * NE];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int u = 0; u < 2; ++u) tra[2 * e + u] = SO::tr_lane(lane) ^ SO::tr_inst(e, u);
  auto slotp = [&](int n) __attribute__((always_inline)) {
    int r = (n % 3) * SLOT;
    opaque(r);
    return r;
  };
  auto rowrd = [&](int base, int st) __attribute__((always_inline)) { return *(const u32x4*)(lds + base + rowa[st]); };
  auto trrd = [&](int base, int t, int e) __attribute__((always_inline)) {
    return cat(lds_read_tr(lds + base + 16 * t * ROWB + tra[2 * e]),
               lds_read_tr(lds + base + (16 * t + 8) * ROWB + tra[2 * e + 1]));
  };

  f32x16 dk[NE], dv[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    dk[e] = zero16();
    dv[e] = zero16();
  }
  const float c2 = a.scale_log2;

  // step n's query block and head
  auto qblock = [&](int n) __attribute__((always_inline)) { return (nqb - 1 - n / G) * BQ; };
  // wave activity and masking for step n (all wave-uniform)
  auto active = [&](int n) __attribute__((always_inline)) { return n < nsteps && (!CAUSAL || kw <= qblock(n)); };
  auto masked = [&](int n) __attribute__((always_inline)) {
    const int qb = qblock(n);
    return (CAUSAL && kw == qb) || qb + BQ > N || kw + 32 > N;
  };

  // S = Q K^T and dP = dO V^T of step n
  auto products = [&](int n, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    const int base = slotp(n);
    s = zero16();
    dp = zero16();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      s = E::mma(rowrd(base, st), kf[st], s);
      dp = E::mma(rowrd(base + TB, st), vf[st], dp);
    }
  };
  // P and dS of step n in place (s -> p, dp -> ds) for elements [lo, hi); rows q = 8(v/4) + 4hh + v%4
  auto elementwise = [&](int base, f32x16& s, f32x16& dp, int lo, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      if (4 * a4 + 3 < lo || 4 * a4 >= hi) continue;
      const f32x4 t0 = *(const f32x4*)(lds + base + 2 * TB + (8 * a4 + 4 * hh) * 8);
      const f32x4 t1 = *(const f32x4*)(lds + base + 2 * TB + (8 * a4 + 4 * hh) * 8 + 16);
      const float l2[4] = {t0[0], t0[2], t1[0], t1[2]}, dd[4] = {t0[1], t0[3], t1[1], t1[3]};
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int v = 4 * a4 + bb;
        if (v < lo || v >= hi) continue;
        const float p = fast_exp2(fmaf(s[v], c2, -l2[bb]));
        s[v] = p;
        dp[v] = p * (dp[v] - dd[bb]);
        keep(s[v]);
        keep(dp[v]);
      }
    }
  };
  auto pack = [&](const f32x16& s, int t) __attribute__((always_inline)) {
    return u32x4{E::pack(s[8 * t + 0], s[8 * t + 1]), E::pack(s[8 * t + 2], s[8 * t + 3]),
                 E::pack(s[8 * t + 4], s[8 * t + 5]), E::pack(s[8 * t + 6], s[8 * t + 7])};
  };
  // dV^T += dO^T P, dK^T += Q^T dS for step n
  auto accumulate = [&](int base, const u32x4* pf, const u32x4* sf) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2 * NE; ++k) {
      const int t = k / NE, e = k % NE;
      dv[e] = E::mma(trrd(base + TB, t, e), pf[t], dv[e]);
      dk[e] = E::mma(trrd(base, t, e), sf[t], dk[e]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step n: the products of step n+1 interleaved with the elementwise work of step n,
  // then (if this wave's keys meet the block at all) the accumulation of step n.  The
  // products of a step past the last, or of one this wave skips, are formed anyway
  // (reading a valid slot) so that every step has the same branch-free core.
  auto step = [&](int n, f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn) __attribute__((always_inline)) {
    if (n > 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads of step n+1 landed
      __syncthreads();                                   // everyone's; slot (n-1)%3 is free
    }
    if (n + 2 < nsteps) dma(n + 2);
    const int bc = slotp(n), bn = slotp(n + 1);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st == 0) {
        sn = zero16();
        dpn = zero16();
      }
      sn = E::mma(rowrd(bn, st), kf[st], sn);
      dpn = E::mma(rowrd(bn + TB, st), vf[st], dpn);
      elementwise(bc, sc, dpc, (16 * st) / NS, (16 * (st + 1)) / NS);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (active(n)) {
      if (masked(n)) {
        const int qb = qblock(n);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = qb + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (q >= N || mykey >= N || (CAUSAL && mykey > q)) {
            sc[v] = 0.f;
            dpc[v] = 0.f;
          }
        }
      }
      const u32x4 pf[2] = {pack(sc, 0), pack(sc, 1)};
      const u32x4 sf[2] = {pack(dpc, 0), pack(dpc, 1)};
      accumulate(bc, pf, sf);
    }
  };

  if (nsteps > 0) {
    dma(0);
    if (nsteps > 1) dma(1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x16 sa, pa, sb, pb;   // S and dP of even / odd steps
  products(0, sa, pa);
  for (int n = 0; n < nsteps; n += 2) {
    step(n, sa, pa, sb, pb);
    if (n + 1 < nsteps) step(n + 1, sb, pb, sa, pa);
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T, rounded to the input dtype
  if (mykey < N) {
    unsigned char* dKg = (unsigned char*)a.dk + (kvhead + mykey) * ROWB;
    unsigned char* dVg = (unsigned char*)a.dv + (kvhead + mykey) * ROWB;
#pragma unroll
    for (int e = 0; e < NE; ++e)
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
  constexpr int PK = ROWB;              // K rows: read by rows (S^T) and transposed (dQ^T): swizzled
  constexpr int PV = ROWB + 16;         // V rows: read by rows (dP^T): padded
  using Tiles = TilePair<ROWB, PK, PV, NW, true>;
  using SO = SwzOffsets<ROWB>;
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
    lse2 = a.rowterm[2 * (qhead + myq)];
    dsv = a.rowterm[2 * (qhead + myq) + 1];
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = df[s] = u32x4{0, 0, 0, 0};
  }

  const int nkv = (N + BC - 1) / BC;
  const int ntile = CAUSAL ? min(nkv, (min(q0 + BR, N) - 1) / BC + 1) : nkv;

  int doff[IPW];
  Tiles::offsets(wave, lane, doff);
  auto dma = [&](int t) __attribute__((always_inline)) { Tiles::load(Kg, Vg, N, t, wave, doff, lds + (t % 3) * SLOT); };

  // per-lane LDS offsets: K rows (swizzled) and V rows (A operands of S^T, dP^T), K
  // transposed (A of dQ^T, swizzled)
  int ka[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) ka[st] = SO::rows_a0(lane) ^ (st << 5);
  int kt[2 * NE];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int u = 0; u < 2; ++u) kt[2 * e + u] = SO::tr_lane(lane) ^ SO::tr_inst(e, u);
  const int va = KBYTES + r32 * PV + 16 * hh;

  const float c2 = a.scale_log2;
  f32x16 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = zero16();

  // unit u = 32 keys = half (u & 1) of tile u >> 1
  auto ubase = [&](int u, int half_pitch) __attribute__((always_inline)) {
    int r = ((u >> 1) % 3) * SLOT + (u & 1) * 32 * half_pitch;
    opaque(r);
    return r;
  };
  auto krow = [&](int kb, int st) __attribute__((always_inline)) { return *(const u32x4*)(lds + kb + ka[st]); };
  auto vrow = [&](int kb, int st) __attribute__((always_inline)) { return *(const u32x4*)(lds + kb + va + 32 * st); };
  auto ktr = [&](int kb, int h, int e) __attribute__((always_inline)) {
    return cat(lds_read_tr(lds + kb + 16 * h * PK + kt[2 * e]), lds_read_tr(lds + kb + (16 * h + 8) * PK + kt[2 * e + 1]));
  };
  // dS of one unit from its S^T and dP^T, packed as the B operand of two 16-key steps
  auto dsfrom = [&](f32x16& s, const f32x16& dp, int lo, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (v >= lo && v < hi) {
        const float p = fast_exp2(fmaf(s[v], c2, -lse2));
        s[v] = p * (dp[v] - dsv);
        keep(s[v]);
      }
  };
  auto pack = [&](const f32x16& s, int h) __attribute__((always_inline)) {
    return u32x4{E::pack(s[8 * h + 0], s[8 * h + 1]), E::pack(s[8 * h + 2], s[8 * h + 3]),
                 E::pack(s[8 * h + 4], s[8 * h + 5]), E::pack(s[8 * h + 6], s[8 * h + 7])};
  };

  const int ulast = (CAUSAL ? min(qw + 31, N - 1) : N - 1) / 32;

  // Unit u < ulast: products of unit u+1 interleaved with the elementwise dS of unit u,
  // then dQ^T += K_u^T dS_u^T.
  auto step_main = [&](int u, f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn) __attribute__((always_inline)) {
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
  auto step_last = [&](int u, f32x16& sc, const f32x16& dpc) __attribute__((always_inline)) {
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

  auto step = [&](int u, f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn) __attribute__((always_inline)) {
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
  auto tile_start = [&](int j) __attribute__((always_inline)) {
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
