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
//  2. dQ pass: one workgroup of 8 waves per (batch, head, 256-query block) — 4 waves
//     and 128 queries, two workgroups per CU, at d = 64 and for small grids — the
//     forward's structure: S^T = K Q^T and dP^T = V dO^T with Q, dO in VGPRs and K
//     (XOR-swizzled: read by rows and transposed), V tiles streamed through LDS;
//     P = exp2(S*scale*log2e - LSE*log2e),
//     dS = P * (dP - D) in registers, dQ^T += K^T dS^T (K read transposed).  d = 64
//     overlaps one unit's elementwise work with the next unit's products; at d = 128 a
//     second unit of S, dP does not fit in the 256 registers of a wave at two waves
//     per SIMD, so each wave takes one unit at a time and the other wave on its SIMD
//     fills the gaps;
//  3. dK/dV pass: one workgroup per (batch, K/V head, 128-key block); each of the
//     4 waves owns 32 keys, holds their K and V in VGPRs and dK^T, dV^T in
//     accumulators across all query heads of the group and all query blocks (from
//     the diagonal when causal; query blocks descending, heads inner, so that
//     concurrent workgroups share Q/dO tiles in L2).  Q, dO and the row terms of each 32-query step go
//     HBM -> LDS directly (three slots, two steps in flight).  Per step:
//     S = Q K^T, dP = dO V^T (lane = key), dV^T += dO^T P, dK^T += Q^T dS (Q^T,
//     dO^T read transposed from LDS); the products of step n+1 are interleaved
//     with the elementwise work of step n.  Where 256-key blocks still give the CUs
//     enough workgroups (512, or 256 without the causal mask), fa_bwd runs instead
//     4 waves x 64 keys (3b below): half the LDS reads per product.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// Row-term layout (the workspace): per (batch, query head), per block of 32 query rows,
// 32 floats LSE_i * log2(e) then 32 floats -D_i; rows of the last block past N hold 0.
__host__ __device__ inline long long rowterm_index(long long bh, int nb32, int row) {
  return (bh * nb32 + row / 32) * 64 + (row & 31);
}

// ---- 1. row terms: LSE_i * log2 e and -D_i = -sum_k dO_ik O_ik per query row ----------
// GEN (the mask family): rows are padded per (batch, head) to ceil(maxq/32) blocks; a
// packed batch takes sequence b's rows from cu_q[b]; a row that saw no key (LSE = -inf)
// stores 0, and all its scores are masked in the passes below.
template <class Tag, int D, bool GEN = false>
__global__ void __launch_bounds__(256) bwd_rowterm_kernel(const BwdArgs a, long long prows) {
  using E = Elt<Tag>;
  constexpr int TPR = D / 8;   // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const int N = a.N;
  const int nb32 = ((GEN ? a.maxq : N) + 31) / 32;
  const long long p = (long long)blockIdx.x * RPB + threadIdx.x / TPR;   // padded row
  const long long bh = p / (32LL * nb32);
  const int r = (int)(p - bh * 32LL * nb32);
  const int part = threadIdx.x % TPR;
  int Lr = N;
  long long row = bh * N + r;
  if constexpr (GEN) {
    if (a.cu_q != nullptr && p < prows) {
      const int b = (int)(bh / a.Hq), h = (int)(bh - (long long)b * a.Hq);
      const int qs = min(max(a.cu_q[b], 0), N), qe = min(max(a.cu_q[b + 1], qs), N);
      Lr = min(qe - qs, a.maxq);
      row = (long long)h * N + qs + r;
    }
  }
  const bool real = p < prows && r < Lr;
  float acc = 0.f;
  if (real) {
    const u32x4 o4 = *(const u32x4*)((const unsigned char*)a.o + (row * D + part * 8) * 2);
    const u32x4 g4 = *(const u32x4*)((const unsigned char*)a.dout + (row * D + part * 8) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(E::to_f32((uint16_t)(o4[i] & 0xffff)), E::to_f32((uint16_t)(g4[i] & 0xffff)), acc);
      acc = fmaf(E::to_f32((uint16_t)(o4[i] >> 16)), E::to_f32((uint16_t)(g4[i] >> 16)), acc);
    }
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, TPR);
  if (p < prows && part == 0) {
    const long long t = rowterm_index(bh, nb32, r);
    const float l = real ? a.lse[row] : 0.f;
    a.rowterm[t] = (real && (!GEN || l > -INFINITY)) ? l * kLog2e : 0.f;
    a.rowterm[t + 32] = real ? -acc : 0.f;
  }
}

// Mask family: sequence b's query and key counts and first rows (0 with fixed lengths);
// offsets are clamped to the tensors.
__device__ __forceinline__ void seq_geometry(const BwdArgs& a, int b, int& Lq, int& Lk, int& qs, int& ks) {
  Lq = a.N;
  Lk = a.Nk;
  qs = ks = 0;
  if (a.cu_q != nullptr) {
    qs = min(max(a.cu_q[b], 0), a.N);
    const int qe = min(max(a.cu_q[b + 1], qs), a.N);
    ks = min(max(a.cu_k[b], 0), a.Nk);
    const int ke = min(max(a.cu_k[b + 1], ks), a.Nk);
    Lq = min(qe - qs, a.maxq);
    Lk = min(ke - ks, a.maxk);
  }
}

// Mask family, dK/dV pass: the 32-query steps [qlo, qtop] (multiples of 32) that hold
// every query whose window meets keys [k0, min(k0 + 128, Lk)); false if no query does.
__device__ __forceinline__ bool dkdv_query_range(const BwdArgs& a, int Lq, int Lk, int k0, int& qlo, int& qtop) {
  const int off = Lk - Lq;   // query i sits at key position i + off
  const int kmax = min(k0 + 128, Lk) - 1;
  const int iq_lo = a.wr >= 0 ? max(k0 - a.wr - off, 0) : 0;
  const int iq_hi = a.wl >= 0 ? min(kmax + a.wl - off, Lq - 1) : Lq - 1;
  qtop = iq_hi >= 0 ? iq_hi / 32 * 32 : 0;
  qlo = iq_lo / 32 * 32;
  return iq_lo <= iq_hi;
}

// ---- block lists, transposed for the dK/dV pass ----------------------------------------
// The lists name, per 256-query block, the 64-key tiles it sees; the dK/dV pass walks a
// 128-key block's queries instead.  One wave per (batch, K/V head, 128-key block) writes
// the runs of 32-query steps that block visits, in the pass's order (query heads of the
// group ascending, query blocks descending): one run per (head, 256-query block) whose
// list holds either of the key block's two tiles, clipped to the queries whose window
// meets the key block.  Record (BwdArgs::rstride ints): [0] runs, [1] steps, then per run
// {first (highest) step's query row, g | steps << 20 | tiles << 28, steps before it},
// tiles bit 0 / bit 1 = the first / second tile listed.  Ballots and lane scans keep the
// order, so the result is the same on every run.
__global__ void __launch_bounds__(256) bwd_runs_kernel(const BwdArgs a, long long nrec, int nkb) {
  const int lane = threadIdx.x & 63;
  const long long rec = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rec >= nrec) return;
  const int jb = (int)(rec % nkb);
  const int grp = (int)(rec / nkb);
  const int b = grp / a.Hkv, hkv = grp - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  int Lq, Lk, qs, ks;
  seq_geometry(a, b, Lq, Lk, qs, ks);
  const int k0 = jb * 128, t0 = k0 / 64;
  int qlo = 0, qtop = 0;
  const bool any = k0 < Lk && dkdv_query_range(a, Lq, Lk, k0, qlo, qtop);
  const int tiles_ok = k0 + 64 < Lk ? 3 : 1;   // the second tile only if it holds keys
  const int nqb = a.bnq, nf = G * nqb;
  int* const out = a.runs + rec * a.rstride;
  int base = 0, steps = 0;
  for (int f0 = 0; any && f0 < nf; f0 += 64) {
    const int f = f0 + lane;
    int tiles = 0, first = 0, nst = 0, g = 0;
    if (f < nf) {
      g = f / nqb;
      const int qb = nqb - 1 - (f - g * nqb);
      const int hi = min(qb * 256 + 224, qtop), lo = max(qb * 256, qlo);
      if (lo <= hi) {
        const int hm = a.bheads == 1 ? 0 : hkv * G + g;
        const size_t row = ((size_t)b * a.bheads + hm) * a.bnq + qb;
        const int cnt = min(max(a.bcnt[row], 0), a.bcap);
        const int* lst = a.bidx + row * a.bcap;
        int p = lower_bound_tiles(lst, cnt, t0);
        if (p < cnt && lst[p] == t0) {
          tiles = 1;
          ++p;
        }
        if (p < cnt && lst[p] == t0 + 1) tiles |= 2;
        tiles &= tiles_ok;
        first = hi;
        nst = (hi - lo) / 32 + 1;
      }
    }
    const unsigned long long m = __ballot(tiles != 0);
    const int pos = base + __popcll(m & ((1ull << lane) - 1));
    const int s = tiles != 0 ? nst : 0;
    int incl = s;   // steps of the kept runs of lanes 0 .. lane
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (tiles != 0) {
      out[2 + 3 * pos] = first;
      out[3 + 3 * pos] = g | (nst << 20) | (tiles << 28);
      out[4 + 3 * pos] = steps + incl - s;
    }
    base += __popcll(m);
    steps += __shfl(incl, 63);
  }
  if (lane == 0) {
    out[0] = base;
    out[1] = steps;
  }
}

// Sum, exclusive prefix sum and maximum over a workgroup of 1024 threads (16 waves), in a
// fixed order; sh holds 16 entries.
template <class T>
__device__ __forceinline__ T wg1024_sum(T v, T* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  T t = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += sh[i];
  __syncthreads();
  return t;
}
__device__ __forceinline__ int wg1024_excl_scan(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += sh[i];
  __syncthreads();
  return off + incl - v;
}
__device__ __forceinline__ int wg1024_max(int v, int* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = sh[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) t = max(t, sh[i]);
  __syncthreads();
  return t;
}

// ---- chunk plan of the transposed lists (one workgroup) ---------------------------------
// Chunk size C = max(kBwdMinChunk, ceil(total steps / kBwdTargetChunks)).  In record
// order, a key block with more than C steps gets ceil(steps / C) chunks and as many
// partial slots while the kBwdSlots last; the rest run whole.  plan[2r] = chunks of record
// r, plan[2r+1] = its first slot; table[0] = slots used, table[1+2s], table[2+2s] = the
// record and chunk of slot s.  Thread t takes a contiguous range of records, so one
// prefix sum orders all of them; the same lists give the same plan.
__global__ void __launch_bounds__(1024) bwd_plan_kernel(const BwdArgs a, int nrec) {
  __shared__ long long shl[16];
  __shared__ int shi[16];
  const int t = threadIdx.x;
  const int per = (nrec + 1023) / 1024;
  const int r0 = min(t * per, nrec), r1 = min(r0 + per, nrec);
  auto steps_of = [&](int r) { return a.runs[(long long)r * a.rstride + 1]; };
  long long mine = 0;
  for (int r = r0; r < r1; ++r) mine += steps_of(r);
  const long long total = wg1024_sum(mine, shl);
  const long long cl = (total + kBwdTargetChunks - 1) / kBwdTargetChunks;
  const int C = (int)max((long long)kBwdMinChunk, cl);
  auto chunks_of = [&](int st) { return st > C ? (st + C - 1) / C : 1; };
  int want = 0;
  for (int r = r0; r < r1; ++r) {
    const int n = chunks_of(steps_of(r));
    want += n > 1 ? n : 0;
  }
  int pos = wg1024_excl_scan(want, shi);
  int used = 0;
  for (int r = r0; r < r1; ++r) {
    const int n = chunks_of(steps_of(r));
    const int w = n > 1 ? n : 0;
    const bool granted = w > 0 && pos + w <= kBwdSlots;
    a.plan[2 * r] = granted ? n : 1;
    a.plan[2 * r + 1] = granted ? pos : 0;
    if (granted) {
      for (int c = 0; c < n; ++c) {
        a.table[1 + 2 * (pos + c)] = r;
        a.table[2 + 2 * (pos + c)] = c;
      }
      used = pos + w;
    }
    pos += w;
  }
  used = wg1024_max(used, shi);
  if (t == 0) a.table[0] = used;
}

// ---- 3. dK, dV per key block ---------------------------------------------------------
// Q rows and dO rows of one 32-query step (XOR-swizzled chunks: lane's 16 bytes of
// tile load i land where soff[i] says) and the step's 256 bytes of row terms, from HBM
// straight into an LDS slot.  qh/gh/rh are the head's first Q row, dO row and row-term
// block; the buffer ranges end at the head's row N, so rows past it arrive as zeros.
// (A free function: the host pass of the compiler mishandles these builtins inside a
// capturing lambda.)
template <int ROWB, int TI, int LI, int NW, int TB>
__device__ __forceinline__ void dkdv_dma(const unsigned char* qh, const unsigned char* gh, const float* rh,
                                         int hbytes, int rbytes, int qoff, int roff, int wave, int lane,
                                         const int* soff, unsigned char* slot) {
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)qh, (short)0, hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)gh, (short)0, hbytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < LI; ++i) {
    const int nn = wave + NW * i;   // tile load: Q for i < LI/2, dO after
    __builtin_amdgcn_raw_ptr_buffer_load_lds(i < LI / 2 ? rq : rd, (lvoid*)(slot + nn * 1024), 16, soff[i] + qoff,
                                             0, 0, 0);
  }
  if (wave == 0) {
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void*)rh, (short)0, rbytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lvoid*)(slot + 2 * TB), 4, lane * 4 + roff, 0, 0, 0);
  }
}

template <class Tag, int D, bool CAUSAL, bool GEN = false, bool SPLIT = false>
__global__ void __launch_bounds__(256) bwd_dkdv_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  using A = AccMma<Tag>;
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
  constexpr int LI = 2 * TI / NW;     // tile loads per wave per step
  constexpr int RT = 2 * TB;          // row terms in the slot: 32 x LSE*log2e, 32 x -D
  constexpr int SLOT = 2 * TB + 256;
  static_assert(TI % NW == 0, "each wave loads whole Q / dO halves");

  // Three slots as distinct LDS objects: with every step's slot known at compile time,
  // the compiler can tell that the loads into one slot do not touch the slots being
  // read, and does not make those reads wait for the loads.
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[SLOT];
  auto slot = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? slot0 : i == 1 ? slot1 : slot2;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;
  const int G = a.Hq / a.Hkv;

  // block -> (key block, batch, kv head): groups x, x+8, ... on XCD x (their Q/dO stay in
  // one L2), key blocks nearest the start (the most causal work) first
  // With block lists, the first kBwdSlots blocks run the chunks of split key blocks (slot
  // table; dealt round-robin over the XCDs and started first, being the long ones), and the
  // primary block of a split key block has nothing to do.
  const int ngroups = a.B * a.Hkv;
  const int nkbg = GEN ? (a.maxk + BKV - 1) / BKV : 0;
  const int nsplit = SPLIT ? a.ksplit : 1;   // fa_bwd: chunks per key block
  int bid = blockIdx.x;
  int jb, grp, chunk = 0;
  bool mapped = false;
  if (GEN && a.plan != nullptr) {
    if (bid < kBwdSlots) {
      if (bid >= a.table[0]) return;
      const int rec = a.table[1 + 2 * bid];
      chunk = a.table[2 + 2 * bid];
      grp = rec / nkbg;
      jb = rec - grp * nkbg;
      mapped = true;
    }
    bid -= kBwdSlots;   // a multiple of 8: the XCD of each primary block is unchanged
  }
  if (!mapped) {   // (the nsplit chunks of a key block follow each other, heaviest blocks first)
    if ((ngroups & 7) == 0) {
      const int x = bid & 7, sidx = bid >> 3, per = ngroups >> 3;
      jb = sidx / (per * nsplit);
      const int rest = sidx - jb * per * nsplit;
      if constexpr (SPLIT) chunk = rest / per;
      grp = x + 8 * (rest - chunk * per);
    } else {
      jb = bid / (ngroups * nsplit);
      const int rest = bid - jb * ngroups * nsplit;
      if constexpr (SPLIT) chunk = rest / ngroups;
      grp = rest - chunk * ngroups;
    }
    if (GEN && a.plan != nullptr && a.plan[2 * (grp * nkbg + jb)] > 1) return;
  }
  const int b = grp / a.Hkv, hkv = grp - b * a.Hkv;
  // sequence geometry: Lq queries, Lk keys; qrow0 = first Q row of query head hkv*G,
  // hs = rows between query heads
  int Lq = N, Lk = N;
  size_t kvhead, qrow0, hs = (size_t)N;
  if constexpr (GEN) {
    int qs, ks;
    seq_geometry(a, b, Lq, Lk, qs, ks);
    if (a.cu_q != nullptr) {
      kvhead = (size_t)hkv * (size_t)a.Nk + ks;
      qrow0 = (size_t)hkv * G * (size_t)N + qs;
    } else {
      kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)a.Nk;
      qrow0 = (size_t)(b * a.Hq + hkv * G) * (size_t)N;
    }
  } else {
    kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
    qrow0 = (size_t)(b * a.Hq + hkv * G) * (size_t)N;
  }
  const int k0 = jb * BKV;
  if (GEN && k0 >= Lk) return;        // the whole workgroup: past this sequence's keys
  const int kw = k0 + 32 * wave;      // first key of this wave
  const int mykey = kw + r32;         // the key this lane's scores belong to
  const int off = Lk - Lq;            // query i sits at key position i + off

  // K^T and V^T as B operands: lane holds row mykey, elements 16s + 8hh .. +7
  u32x4 kf[NS], vf[NS];
  if (mykey < Lk) {
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

  // Steps: for each query head of the group, query blocks from the last down to the
  // first one that meets these keys (the key block's own start when causal; under a
  // window, the blocks of queries whose window meets the block's keys; with block lists,
  // only the runs of steps the transposed lists name).
  const int nb32 = ((GEN ? a.maxq : N) + 31) / 32;
  int qtop, qlo, nsteps;
  const int* runs = nullptr;
  int nruns = 0, run0 = 0, skip0 = 0;   // with lists: the chunk starts skip0 steps into run run0
  int nchunk = 1, pslot = 0;            // chunks of this key block, this chunk's partial slot
  int s0 = 0;                           // fa_bwd split: this chunk's first step
  if constexpr (GEN) {
    static_assert(BKV == 128 && BQ == 32, "dkdv_query_range and the runs assume these");
    const bool any = dkdv_query_range(a, Lq, Lk, k0, qlo, qtop);
    if (a.runs != nullptr) {
      const int rec = grp * nkbg + jb;
      runs = a.runs + (long long)rec * a.rstride;
      nruns = runs[0];
      const int steps = runs[1];
      nchunk = a.plan[2 * rec];
      pslot = a.plan[2 * rec + 1] + chunk;
      const int per = (steps + nchunk - 1) / nchunk;
      const int s0 = min(chunk * per, steps);
      nsteps = min(s0 + per, steps) - s0;
      if (nsteps > 0) {   // the last run that starts at or before step s0
        int lo = 0, hi = nruns - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (runs[4 + 3 * mid] <= s0) lo = mid;
          else hi = mid - 1;
        }
        run0 = lo;
        skip0 = s0 - runs[4 + 3 * lo];
      }
    } else {
      nsteps = any ? G * ((qtop - qlo) / BQ + 1) : 0;
    }
  } else {
    qtop = (nb32 - 1) * BQ;
    qlo = CAUSAL ? k0 : 0;
    nsteps = G * ((qtop - qlo) / BQ + 1);
    if (SPLIT) {   // this chunk's steps [s0, s0 + nsteps) of the key block's sequence
      const int total = nsteps, per = (total + nsplit - 1) / nsplit;
      s0 = min(chunk * per, total);
      nsteps = min(s0 + per, total) - s0;
      nchunk = nsplit;
      pslot = (grp * ((N + BKV - 1) / BKV) + jb) * nsplit + chunk;
    }
  }

  // ---- HBM -> LDS (step n into slot n % 3), driven by a cursor over (head, block) ----
  int soff[LI];
#pragma unroll
  for (int i = 0; i < LI; ++i) {
    const int nn = wave + NW * i;
    const int row = (nn % TI) * RPI + lane / CH;
    soff[i] = row * ROWB + (((lane % CH) ^ swz<CH>(row)) << 4);
  }
  const unsigned char* const q_g = (const unsigned char*)a.q + qrow0 * ROWB;
  const unsigned char* const g_g = (const unsigned char*)a.dout + qrow0 * ROWB;
  const float* const r_g = a.rowterm + (long long)(b * a.Hq + hkv * G) * nb32 * 64;
  const unsigned char* dq_h = q_g;
  const unsigned char* dg_h = g_g;
  const float* dr_h = r_g;
  const int hbytes = Lq * ROWB, rbytes = nb32 * 256;   // buffer ranges: rows past Lq read 0
  int dqb = qtop;   // query block of the next step to load
  if (SPLIT && s0 > 0) {   // a later chunk: start s0 steps in (heads outer, blocks descending)
    const int spb = (qtop - qlo) / BQ + 1, g0 = s0 / spb;
    dqb = qtop - BQ * (s0 - g0 * spb);
    dq_h += (size_t)g0 * hs * ROWB;
    dg_h += (size_t)g0 * hs * ROWB;
    dr_h += (long long)g0 * nb32 * 64;
  }
  // block lists: run dri of the records, steps left in it, its tiles
  int dri = 0, dleft = 0, dtiles = 3;
  auto load_run = [&](int r) __attribute__((always_inline)) {
    dqb = runs[2 + 3 * r];
    const int w = runs[3 + 3 * r];
    const int g = w & 0xfffff;
    dleft = (w >> 20) & 15;
    dtiles = (w >> 28) & 3;
    dq_h = q_g + g * hs * ROWB;
    dg_h = g_g + g * hs * ROWB;
    dr_h = r_g + (long long)g * nb32 * 64;
  };
  // GEN: the query block and tiles of the step loaded into each slot
  int sqb[3], stiles[3];
  auto dma_next = [&](unsigned char* sl, int si) __attribute__((always_inline)) {
    dkdv_dma<ROWB, TI, LI, NW, TB>(dq_h, dg_h, dr_h, hbytes, rbytes, dqb * ROWB, dqb * 8, wave, lane, soff, sl);
    if constexpr (GEN) {
      sqb[si] = dqb;
      stiles[si] = dtiles;
    }
    dqb -= BQ;
    if (GEN && runs != nullptr) {
      if (--dleft == 0 && ++dri < nruns) load_run(dri);
    } else if (dqb < qlo) {
      dqb = qtop;
      dq_h += hs * ROWB;
      dg_h += hs * ROWB;
      dr_h += nb32 * 64;
    }
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
  auto rowrd = [&](const unsigned char* sl, int st) __attribute__((always_inline)) {
    return *(const u32x4*)(sl + rowa[st]);
  };
  auto trrd = [&](const unsigned char* sl, int t, int e) __attribute__((always_inline)) {
    return cat(lds_read_tr(sl + 16 * t * ROWB + tra[2 * e]), lds_read_tr(sl + (16 * t + 8) * ROWB + tra[2 * e + 1]));
  };
  // row terms of this lane's 16 rows q = 8(v/4) + 4hh + v%4: four 16-byte reads
  auto rt4 = [&](const unsigned char* sl, int off, int j) __attribute__((always_inline)) {
    return *(const f32x4*)(sl + RT + off + (8 * j + 4 * hh) * 4);
  };
  auto rt16 = [&](const unsigned char* sl, int off) __attribute__((always_inline)) {
    f32x16 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 t = rt4(sl, off, j);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[4 * j + i] = t[i];
    }
    return r;
  };

  f32x16 dk[NE], dv[NE];
  acc_init(dk);
  acc_init(dv);
  const float c2 = a.scale_log2;

  auto pack = [&](const f32x16& s, int t) __attribute__((always_inline)) {
    return u32x4{E::pack(s[8 * t + 0], s[8 * t + 1]), E::pack(s[8 * t + 2], s[8 * t + 3]),
                 E::pack(s[8 * t + 4], s[8 * t + 5]), E::pack(s[8 * t + 6], s[8 * t + 7])};
  };

  // Step n (slot J % 3; S, dP of step n in (sc, dpc), of step n+1 formed into (sn, dpn)):
  //   sync; load step n+2;
  //   NS sub-steps: [elementwise of step n: P = exp2(S*c - LSE2), dS = P * (dP - D)]
  //                 [S_{n+1} += Q K^T, dP_{n+1} += dO V^T for one k-step]
  //   if the step meets this wave's keys: (diagonal: mask) pack; dV^T += dO^T P,
  //   dK^T += Q^T dS.
  // dP_{n+1} starts from -D, so dP - D comes out of the MFMA.  The products of a step
  // past the last are formed anyway from a valid slot and never used.
  int cqb_plain = dqb;    // query block of the current step (GEN: recorded per slot)
  f32x16 l2n;             // LSE*log2e of the current step's rows
  auto step = [&](auto Jc, int n, f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn) __attribute__((always_inline)) {
    constexpr int J = decltype(Jc)::value;
    unsigned char* const bc = slot(J % 3);
    unsigned char* const bn = slot((J + 1) % 3);
    unsigned char* const bl = slot((J + 2) % 3);
    if (n > 0) {
      wait_loads();      // this wave's loads of step n+1 landed
      __syncthreads();   // everyone's; everyone is done with slot (n-1)%3
    }
    if (n + 2 < nsteps) dma_next(bl, (J + 2) % 3);
    const f32x16 l2 = l2n;
    const f32x16 nd = rt16(bn, 128);
    u32x4 qa = rowrd(bn, 0), ga = rowrd(bn + TB, 0);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
#pragma unroll
      for (int v = (16 * st) / NS; v < (16 * (st + 1)) / NS; ++v) {
        const float p = fast_exp2(fmaf(sc[v], c2, -l2[v]));
        sc[v] = p;
        dpc[v] = p * dpc[v];
        keep(sc[v]);
        keep(dpc[v]);
      }
      const u32x4 qc = qa, gc = ga;
      if (st + 1 < NS) {
        qa = rowrd(bn, st + 1);
        ga = rowrd(bn + TB, st + 1);
      }
      sn = E::mma(qc, kf[st], st == 0 ? zero16() : sn);
      dpn = E::mma(gc, vf[st], st == 0 ? nd : dpn);
      __builtin_amdgcn_sched_barrier(0);
    }
    l2n = rt16(bn, 0);
    bool active, full;
    int cqb;   // the step's first query
    if constexpr (GEN) {
      cqb = sqb[J % 3];
      // wave-uniform: does any (query, key) pair of this step and wave meet, do all?
      // (with block lists, only if the list names this wave's tile)
      const int qmax = min(cqb + BQ, Lq) - 1, kmax = min(kw + 32, Lk) - 1;
      const int vlo = a.wl >= 0 ? cqb + off - a.wl : 0;              // keys some query sees
      const int vhi = a.wr >= 0 ? qmax + off + a.wr : Lk - 1;
      active = kw <= kmax && cqb <= qmax && max(vlo, kw) <= min(vhi, kmax) && ((stiles[J % 3] >> (wave >> 1)) & 1);
      full = kw + 31 < Lk && cqb + BQ - 1 < Lq && (a.wl < 0 || qmax + off - a.wl <= kw) &&
             (a.wr < 0 || kw + 31 <= cqb + off + a.wr);
    } else {
      cqb = cqb_plain;
      active = !CAUSAL || cqb >= kw;
      full = !CAUSAL || cqb != kw;
    }
    if (active) {
      if (!full) {
        // query cqb + 8(v/4) + 4hh + v%4 against this lane's key: outside the mask -> 0
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int qi = cqb + 8 * (v >> 2) + 4 * hh + (v & 3);
          bool vis;
          if constexpr (GEN)
            vis = qi < Lq && mykey < Lk && (a.wl < 0 || mykey >= qi + off - a.wl) &&
                  (a.wr < 0 || mykey <= qi + off + a.wr);
          else
            vis = mykey <= qi;
          if (!vis) {
            sc[v] = 0.f;
            dpc[v] = 0.f;
          }
        }
      }
      const u32x4 pf[2] = {pack(sc, 0), pack(sc, 1)};
      const u32x4 sf[2] = {pack(dpc, 0), pack(dpc, 1)};
      keep(pf[0]);
      keep(pf[1]);
      keep(sf[0]);
      keep(sf[1]);
      u32x4 ta = trrd(bc + TB, 0, 0), tb = trrd(bc, 0, 0);
#pragma unroll
      for (int k = 0; k < 2 * NE; ++k) {
        const int t = k / NE, e = k % NE;
        const u32x4 tc = ta, td = tb;
        if (k + 1 < 2 * NE) {
          ta = trrd(bc + TB, (k + 1) / NE, (k + 1) % NE);
          tb = trrd(bc, (k + 1) / NE, (k + 1) % NE);
        }
        if (k == 0) {
          A::mma_fresh(dv[e], tc, pf[t]);
          A::mma_fresh(dk[e], td, sf[t]);
        } else {
          A::mma(dv[e], tc, pf[t]);
          A::mma(dk[e], td, sf[t]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!GEN) {
      cqb_plain -= BQ;
      if (cqb_plain < qlo) cqb_plain = qtop;
    }
  };

  if (nsteps > 0) {
    if (GEN && runs != nullptr) {
      dri = run0;
      load_run(run0);
      dqb -= BQ * skip0;
      dleft -= skip0;
    }
    dma_next(slot0, 0);
    if (nsteps > 1) dma_next(slot1, 1);
  }
  wait_loads();
  __syncthreads();
  f32x16 sa, pa, sb, pb;   // S and dP of even / odd steps
  {
    const f32x16 nd = rt16(slot0, 128);
    sa = zero16();
    pa = nd;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      sa = E::mma(rowrd(slot0, st), kf[st], sa);
      pa = E::mma(rowrd(slot0 + TB, st), vf[st], pa);
    }
    l2n = rt16(slot0, 0);
  }
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  for (int n = 0; n < nsteps; n += 6) {
    step(I0{}, n, sa, pa, sb, pb);
    if (n + 1 >= nsteps) break;
    step(I1{}, n + 1, sb, pb, sa, pa);
    if (n + 2 >= nsteps) break;
    step(I2{}, n + 2, sa, pa, sb, pb);
    if (n + 3 >= nsteps) break;
    step(I3{}, n + 3, sb, pb, sa, pa);
    if (n + 4 >= nsteps) break;
    step(I4{}, n + 4, sa, pa, sb, pb);
    if (n + 5 >= nsteps) break;
    step(I5{}, n + 5, sb, pb, sa, pa);
  }
  acc_drain(dk);
  acc_drain(dv);

  if ((GEN || SPLIT) && nchunk > 1) {
    // one chunk of a split key block: fp32 partial dK^T (unscaled), dV^T as [key][d]
    float* pk = a.pool + (size_t)pslot * 2 * BKV * D + (size_t)(32 * wave + r32) * D;
    float* pv = pk + BKV * D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * e + 8 * g4 + 4 * hh;
        *(f32x4*)(pk + d0) = f32x4{dk[e][4 * g4], dk[e][4 * g4 + 1], dk[e][4 * g4 + 2], dk[e][4 * g4 + 3]};
        *(f32x4*)(pv + d0) = f32x4{dv[e][4 * g4], dv[e][4 * g4 + 1], dv[e][4 * g4 + 2], dv[e][4 * g4 + 3]};
      }
    return;
  }

  // dK = scale * (dK^T)^T, dV = (dV^T)^T, rounded to the input dtype
  if (mykey < Lk) {   // (both lanes of a key take this together)
    store_row16<E>((unsigned char*)a.dk + (kvhead + mykey) * ROWB, dk, a.scale, hh);
    store_row16<E>((unsigned char*)a.dv + (kvhead + mykey) * ROWB, dv, 1.f, hh);
  }
}

// ---- 3b. dK, dV with 64 keys per wave (fa_bwd where the 256-key grid fills the CUs) -----
// Four waves x 64 keys: each wave holds K and V of two 32-key halves and their dK^T, dV^T
// (all 256 accumulator registers), so every Q / dO operand read from LDS feeds two
// products, half the LDS bytes per product of the 32-key pass, whose one wave per SIMD
// cannot pull more LDS bandwidth than it uses.  No room is left for a software pipeline;
// instead each step orders its work so that the vector ALU runs under the matrix cores:
// the S products; the dP products, each slot with a share of P's exponentials; the dV
// products (they need only P), each slot with a share of dS = P * (dP - D); the dK
// products.  Per key, the same operations in the same order as the 32-key pass (steps a
// wave cannot see add nothing), so both give the same bits.
template <class Tag, int D, bool CAUSAL, bool SPLIT = false>
__global__ void __launch_bounds__(256) bwd_dkdv64_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  using A = AccMma<Tag>;
  constexpr int NW = 4;
  constexpr int KW = 64;
  constexpr int BKV = KW * NW;
  constexpr int BQ = 32;
  constexpr int ROWB = D * 2;
  constexpr int CH = D / 8;
  constexpr int NS = D / 16;
  constexpr int NE = D / 32;
  constexpr int TB = BQ * ROWB;
  constexpr int TI = TB / 1024;
  constexpr int RPI = 1024 / ROWB;
  constexpr int LI = 2 * TI / NW;
  constexpr int RT = 2 * TB;
  constexpr int SLOT = 2 * TB + 256;
  static_assert(TI % NW == 0, "each wave loads whole Q / dO halves");
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[SLOT];
  auto slot = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? slot0 : i == 1 ? slot1 : slot2;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;
  const int G = a.Hq / a.Hkv;
  // block -> (key block, chunk, batch, K/V head) as in the 32-key pass
  const int ngroups = a.B * a.Hkv;
  const int nsplit = SPLIT ? a.ksplit : 1;
  const int bid = blockIdx.x;
  int jb, grp, chunk = 0;
  if ((ngroups & 7) == 0) {
    const int x = bid & 7, sidx = bid >> 3, per = ngroups >> 3;
    jb = sidx / (per * nsplit);
    const int rest = sidx - jb * per * nsplit;
    if constexpr (SPLIT) chunk = rest / per;
    grp = x + 8 * (rest - chunk * per);
  } else {
    jb = bid / (ngroups * nsplit);
    const int rest = bid - jb * ngroups * nsplit;
    if constexpr (SPLIT) chunk = rest / ngroups;
    grp = rest - chunk * ngroups;
  }
  const int b = grp / a.Hkv, hkv = grp - b * a.Hkv;
  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
  const size_t qrow0 = (size_t)(b * a.Hq + hkv * G) * (size_t)N;
  const size_t hs = (size_t)N;
  const int k0 = jb * BKV;
  const int kw = k0 + KW * wave;
  u32x4 kf[2][NS], vf[2][NS];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = kw + 32 * h + r32;
    if (key < N) {
      const unsigned char* kp = (const unsigned char*)a.k + (kvhead + key) * ROWB + 16 * hh;
      const unsigned char* vp = (const unsigned char*)a.v + (kvhead + key) * ROWB + 16 * hh;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        kf[h][st] = *(const u32x4*)(kp + 32 * st);
        vf[h][st] = *(const u32x4*)(vp + 32 * st);
      }
    } else {
#pragma unroll
      for (int st = 0; st < NS; ++st) kf[h][st] = vf[h][st] = u32x4{0, 0, 0, 0};
    }
  }
  const int nb32 = (N + 31) / 32;
  const int qtop = (nb32 - 1) * BQ;
  const int qlo = CAUSAL ? k0 : 0;
  int nsteps = G * ((qtop - qlo) / BQ + 1);
  int s0 = 0;
  if constexpr (SPLIT) {   // this chunk's steps [s0, s0 + nsteps)
    const int total = nsteps, per = (total + nsplit - 1) / nsplit;
    s0 = min(chunk * per, total);
    nsteps = min(s0 + per, total) - s0;
  }
  int soff[LI];
#pragma unroll
  for (int i = 0; i < LI; ++i) {
    const int nn = wave + NW * i;
    const int row = (nn % TI) * RPI + lane / CH;
    soff[i] = row * ROWB + (((lane % CH) ^ swz<CH>(row)) << 4);
  }
  const unsigned char* dq_h = (const unsigned char*)a.q + qrow0 * ROWB;
  const unsigned char* dg_h = (const unsigned char*)a.dout + qrow0 * ROWB;
  const float* dr_h = a.rowterm + (long long)(b * a.Hq + hkv * G) * nb32 * 64;
  const int hbytes = N * ROWB, rbytes = nb32 * 256;
  int dqb = qtop;
  if (SPLIT && s0 > 0) {   // a later chunk: start s0 steps in (heads outer, blocks descending)
    const int spb = (qtop - qlo) / BQ + 1, g0 = s0 / spb;
    dqb = qtop - BQ * (s0 - g0 * spb);
    dq_h += (size_t)g0 * hs * ROWB;
    dg_h += (size_t)g0 * hs * ROWB;
    dr_h += (long long)g0 * nb32 * 64;
  }
  int sqb[3];
  auto dma_next = [&](unsigned char* sl, int si) __attribute__((always_inline)) {
    dkdv_dma<ROWB, TI, LI, NW, TB>(dq_h, dg_h, dr_h, hbytes, rbytes, dqb * ROWB, dqb * 8, wave, lane, soff, sl);
    sqb[si] = dqb;
    dqb -= BQ;
    if (dqb < qlo) {
      dqb = qtop;
      dq_h += hs * ROWB;
      dg_h += hs * ROWB;
      dr_h += nb32 * 64;
    }
  };
  using SO = SwzOffsets<ROWB>;
  const int ra0 = SO::rows_a0(lane);
  const int trl = SO::tr_lane(lane);
  auto rowrd = [&](const unsigned char* sl, int st) __attribute__((always_inline)) {
    return *(const u32x4*)(sl + (ra0 ^ (st << 5)));
  };
  auto trrd = [&](const unsigned char* sl, int t, int e) __attribute__((always_inline)) {
    return cat(lds_read_tr(sl + 16 * t * ROWB + (trl ^ SO::tr_inst(e, 0))),
               lds_read_tr(sl + (16 * t + 8) * ROWB + (trl ^ SO::tr_inst(e, 1))));
  };
  auto rt16 = [&](const unsigned char* sl, int off) __attribute__((always_inline)) {
    f32x16 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 t = *(const f32x4*)(sl + RT + off + (8 * j + 4 * hh) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[4 * j + i] = t[i];
    }
    return r;
  };
  auto pack = [&](const f32x16& x, int t) __attribute__((always_inline)) {
    return u32x4{E::pack(x[8 * t + 0], x[8 * t + 1]), E::pack(x[8 * t + 2], x[8 * t + 3]),
                 E::pack(x[8 * t + 4], x[8 * t + 5]), E::pack(x[8 * t + 6], x[8 * t + 7])};
  };
  f32x16 dk0[NE], dk1[NE], dv0[NE], dv1[NE];
  acc_init(dk0);
  acc_init(dk1);
  acc_init(dv0);
  acc_init(dv1);
  const float c2 = a.scale_log2;
  // S products; then the dP products, each slot with four of P's exponentials; then the dV
  // products (they need only P), each slot with four of dS's products; then the dK products
  auto step = [&](auto Sc) __attribute__((always_inline)) {
    constexpr int SI = decltype(Sc)::value;
    unsigned char* const bc = slot(SI);
    const int cqb = sqb[SI];
    if (CAUSAL && cqb + BQ - 1 < kw) return;   // every query of the step before every key of the wave
    f32x16 s0, s1, p0, p1;
    {
      u32x4 qa = rowrd(bc, 0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const u32x4 qc = qa;
        if (st + 1 < NS) qa = rowrd(bc, st + 1);
        s0 = E::mma(qc, kf[0][st], st == 0 ? zero16() : s0);
        s1 = E::mma(qc, kf[1][st], st == 0 ? zero16() : s1);
      }
    }
    const bool diag = CAUSAL && cqb < kw + KW - 1;
    {
      const f32x16 l2 = rt16(bc, 0);
      const f32x16 nd = rt16(bc, 128);
      u32x4 ga = rowrd(bc + TB, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const u32x4 gc = ga;
        if (st + 1 < NS) ga = rowrd(bc + TB, st + 1);
#pragma unroll
        for (int v = (16 * st) / NS; v < (16 * (st + 1)) / NS; ++v) {
          s0[v] = fast_exp2(fmaf(s0[v], c2, -l2[v]));
          s1[v] = fast_exp2(fmaf(s1[v], c2, -l2[v]));
          keep(s0[v]);
          keep(s1[v]);
        }
        p0 = E::mma(gc, vf[0][st], st == 0 ? nd : p0);
        p1 = E::mma(gc, vf[1][st], st == 0 ? nd : p1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (diag) {   // query cqb + 8(v/4) + 4hh + v%4 before the key: P = 0
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int qi = cqb + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (kw + r32 > qi) s0[v] = 0.f;
        if (kw + 32 + r32 > qi) s1[v] = 0.f;
      }
    }
    const u32x4 pf0[2] = {pack(s0, 0), pack(s0, 1)};
    const u32x4 pf1[2] = {pack(s1, 0), pack(s1, 1)};
    keep(pf0[0]);
    keep(pf0[1]);
    keep(pf1[0]);
    keep(pf1[1]);
    __builtin_amdgcn_sched_barrier(0);
    {
      u32x4 ta = trrd(bc + TB, 0, 0);
#pragma unroll
      for (int k = 0; k < 2 * NE; ++k) {
        const u32x4 tc = ta;
        if (k + 1 < 2 * NE) ta = trrd(bc + TB, (k + 1) / NE, (k + 1) % NE);
#pragma unroll
        for (int v = (16 * k) / (2 * NE); v < (16 * (k + 1)) / (2 * NE); ++v) {
          p0[v] = s0[v] * p0[v];
          p1[v] = s1[v] * p1[v];
          keep(p0[v]);
          keep(p1[v]);
        }
        if (k == 0) A::mma_fresh(dv0[k % NE], tc, pf0[k / NE]);
        else A::mma(dv0[k % NE], tc, pf0[k / NE]);
        A::mma(dv1[k % NE], tc, pf1[k / NE]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const u32x4 sf0[2] = {pack(p0, 0), pack(p0, 1)};
    const u32x4 sf1[2] = {pack(p1, 0), pack(p1, 1)};
    keep(sf0[0]);
    keep(sf0[1]);
    keep(sf1[0]);
    keep(sf1[1]);
    __builtin_amdgcn_sched_barrier(0);
    {
      u32x4 tb = trrd(bc, 0, 0);
#pragma unroll
      for (int k = 0; k < 2 * NE; ++k) {
        const u32x4 td = tb;
        if (k + 1 < 2 * NE) tb = trrd(bc, (k + 1) / NE, (k + 1) % NE);
        if (k == 0) A::mma_fresh(dk0[k % NE], td, sf0[k / NE]);
        else A::mma(dk0[k % NE], td, sf0[k / NE]);
        A::mma(dk1[k % NE], td, sf1[k / NE]);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  auto iter = [&](auto Jc, int n) __attribute__((always_inline)) {
    constexpr int J = decltype(Jc)::value;
    if (n > 0) {
      wait_loads();
      __syncthreads();
    }
    if (n + 2 < nsteps) dma_next(slot((J + 2) % 3), (J + 2) % 3);
    step(Jc);
  };
  if (nsteps > 0) {
    dma_next(slot0, 0);
    if (nsteps > 1) dma_next(slot1, 1);
    wait_loads();
    __syncthreads();
    for (int n = 0; n < nsteps; n += 3) {
      iter(I0{}, n);
      if (n + 1 >= nsteps) break;
      iter(I1{}, n + 1);
      if (n + 2 >= nsteps) break;
      iter(I2{}, n + 2);
    }
  }
  acc_drain(dk0);
  acc_drain(dk1);
  acc_drain(dv0);
  acc_drain(dv1);
  auto store = [&](const f32x16 (&dk)[NE], const f32x16 (&dv)[NE], int key) __attribute__((always_inline)) {
    if (key >= N) return;
    store_row16<E>((unsigned char*)a.dk + (kvhead + key) * ROWB, dk, a.scale, hh);
    store_row16<E>((unsigned char*)a.dv + (kvhead + key) * ROWB, dv, 1.f, hh);
  };
  if constexpr (SPLIT) {
    if (nsplit > 1) {   // fp32 partial dK^T (unscaled) then dV^T of the 256 keys, as [key][d]
      const int pslot = (grp * ((N + BKV - 1) / BKV) + jb) * nsplit + chunk;
      float* pk = a.pool + (size_t)pslot * 2 * BKV * D;
      auto part = [&](const f32x16 (&acc)[NE], float* base, int lkey) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * e + 8 * g4 + 4 * hh;
            *(f32x4*)(base + (size_t)lkey * D + d0) =
                f32x4{acc[e][4 * g4], acc[e][4 * g4 + 1], acc[e][4 * g4 + 2], acc[e][4 * g4 + 3]};
          }
      };
      part(dk0, pk, KW * wave + r32);
      part(dk1, pk, KW * wave + 32 + r32);
      part(dv0, pk + BKV * D, KW * wave + r32);
      part(dv1, pk + BKV * D, KW * wave + 32 + r32);
      return;
    }
  }
  store(dk0, dv0, kw + r32);
  store(dk1, dv1, kw + 32 + r32);
}

// ---- sum of the partial dK, dV of split key blocks ----------------------------------------
// One workgroup per slot: the slot of chunk c of a key block split n ways takes keys
// [128c/n, 128(c+1)/n) of the block, sums the n partials (consecutive slots) in chunk
// order and writes dK = scale * sum, dV = sum in the input dtype.
// Without a slot table (fa_bwd's split): record `rec` (a.kblock keys) owns slots
// rec*ksplit .. rec*ksplit + ksplit - 1.
template <class Tag, int D>
__global__ void __launch_bounds__(256) bwd_reduce_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  constexpr int ROWB = D * 2;
  int c, sl, rec, n, jb, Lk, kb = 128;   // chunk, chunk 0's slot, record, chunks, key block, keys, keys a record
  size_t kvhead;
  if (a.table != nullptr) {
    if ((int)blockIdx.x >= a.table[0]) return;
    c = a.table[2 + 2 * blockIdx.x];
    sl = blockIdx.x - c;
    rec = a.table[1 + 2 * blockIdx.x];
    const int nkbg = (a.maxk + 127) / 128;
    const int grp = rec / nkbg;
    jb = rec - grp * nkbg;
    const int b = grp / a.Hkv, hkv = grp - b * a.Hkv;
    int Lq, qs, ks;
    seq_geometry(a, b, Lq, Lk, qs, ks);
    kvhead = a.cu_q != nullptr ? (size_t)hkv * (size_t)a.Nk + ks : (size_t)(b * a.Hkv + hkv) * (size_t)a.Nk;
    n = a.plan[2 * rec];
  } else {
    n = a.ksplit;
    kb = a.kblock;
    rec = blockIdx.x / n;
    c = blockIdx.x - rec * n;
    sl = rec * n;
    const int nkb = (a.N + kb - 1) / kb;
    const int grp = rec / nkb;
    jb = rec - grp * nkb;
    Lk = a.N;
    kvhead = (size_t)grp * (size_t)a.N;   // grp = batch * Hkv + K/V head
  }
  const int k0 = jb * kb;
  const int key0 = kb * c / n, nk = kb * (c + 1) / n - key0;
  for (int i = threadIdx.x; i < 2 * nk * (D / 8); i += 256) {
    const int t = i / (nk * (D / 8));   // 0: dK, 1: dV
    const int e8 = i - t * nk * (D / 8);
    const int key = key0 + e8 / (D / 8), d0 = (e8 % (D / 8)) * 8;
    if (k0 + key >= Lk) continue;
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < n; ++c) {
      const float* p = a.pool + ((size_t)(sl + c) * 2 + t) * kb * D + (size_t)key * D + d0;
      lo += *(const f32x4*)p;
      hi += *(const f32x4*)(p + 4);
    }
    const float m = t == 0 ? a.scale : 1.f;
    const u32x4 w = {E::pack(lo[0] * m, lo[1] * m), E::pack(lo[2] * m, lo[3] * m), E::pack(hi[0] * m, hi[1] * m),
                     E::pack(hi[2] * m, hi[3] * m)};
    unsigned char* out = (unsigned char*)(t == 0 ? a.dk : a.dv) + (kvhead + k0 + key) * ROWB + d0 * 2;
    *(u32x4*)out = w;
  }
}

// ---- 2. dQ per query block -------------------------------------------------------------
// PIPE: the next unit's products interleaved with this unit's elementwise work (two
// units of S, dP live at once); otherwise one unit at a time.
template <class Tag, int D, bool CAUSAL, int NW, bool PIPE, bool GEN = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) bwd_dq_kernel(const BwdArgs a) {
  using E = Elt<Tag>;
  using A = AccMma<Tag>;
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

  // NSL slots as distinct LDS objects (see the dK/dV pass): tile j uses slot j % NSL,
  // known at compile time in the NSL-tile unrolled loops.  Three (two tiles in flight)
  // unless two 4-wave workgroups must share a CU at d = 128 (33 KB a slot).
  constexpr int NSL = (D == 128 && NW < 8) ? 2 : 3;
  static_assert(!PIPE || NSL == 3, "the pipeline reads the next tile before its barrier");
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[NSL == 3 ? SLOT : 1];
  auto slot = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? slot0 : i == 1 ? slot1 : slot2;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;

  int b, hq, iq;
  map_q_block(((GEN ? a.maxq : N) + BR - 1) / BR, a.B, a.Hq, a.Hkv, b, hq, iq);
  const int hkv = hq / (a.Hq / a.Hkv);
  int Lq = N, Lk = N;
  size_t qhead, kvhead;
  if constexpr (GEN) {
    if (a.cu_q != nullptr) {
      const int qs = min(max(a.cu_q[b], 0), N), qe = min(max(a.cu_q[b + 1], qs), N);
      const int ks = min(max(a.cu_k[b], 0), a.Nk), ke = min(max(a.cu_k[b + 1], ks), a.Nk);
      Lq = min(qe - qs, a.maxq);
      Lk = min(ke - ks, a.maxk);
      qhead = (size_t)hq * (size_t)N + qs;
      kvhead = (size_t)hkv * (size_t)a.Nk + ks;
    } else {
      Lk = a.Nk;
      qhead = (size_t)(b * a.Hq + hq) * (size_t)N;
      kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)a.Nk;
    }
  } else {
    qhead = (size_t)(b * a.Hq + hq) * (size_t)N;
    kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
  }
  const unsigned char* Kg = (const unsigned char*)a.k + kvhead * ROWB;
  const unsigned char* Vg = (const unsigned char*)a.v + kvhead * ROWB;

  const int q0 = iq * BR;
  if (GEN && q0 >= Lq) return;         // the whole workgroup: past this sequence's queries
  const int qw = q0 + wave * 32;
  const int myq = qw + r32;            // the query this lane's scores belong to
  const int off = Lk - Lq;

  // Q^T and dO^T as B operands: lane holds row myq, elements 16s + 8hh .. +7
  u32x4 qf[NS], df[NS];
  float lse2 = 0.f, negd = 0.f;
  if (myq < Lq) {
    const unsigned char* qp = (const unsigned char*)a.q + (qhead + myq) * ROWB + 16 * hh;
    const unsigned char* gp = (const unsigned char*)a.dout + (qhead + myq) * ROWB + 16 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qf[s] = *(const u32x4*)(qp + 32 * s);
      df[s] = *(const u32x4*)(gp + 32 * s);
    }
    if (GEN || !a.rowterm_here) {
      const long long t = rowterm_index((long long)b * a.Hq + hq, ((GEN ? a.maxq : N) + 31) / 32, myq);
      lse2 = a.rowterm[t];
      negd = a.rowterm[t + 32];
    } else {
      // the row terms of fa_bwd formed here, for this pass and (written below) the dK/dV
      // pass: D in the row-term kernel's order (each 8-element part summed in sequence,
      // then the parts pairwise: the partner half-wave, then s ^ 1, s ^ 2, s ^ 4)
      const unsigned char* op = (const unsigned char*)a.o + (qhead + myq) * ROWB + 16 * hh;
      float part[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 o4 = *(const u32x4*)(op + 32 * s), g4 = df[s];
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = fmaf(E::to_f32((uint16_t)(o4[i] & 0xffff)), E::to_f32((uint16_t)(g4[i] & 0xffff)), acc);
          acc = fmaf(E::to_f32((uint16_t)(o4[i] >> 16)), E::to_f32((uint16_t)(g4[i] >> 16)), acc);
        }
        part[s] = half_sum(acc);
      }
#pragma unroll
      for (int w = 1; w < NS; w <<= 1)
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if ((s & w) == 0 && (s & (w - 1)) == 0) part[s] = part[s] + part[s + w];
      lse2 = a.lse[qhead + myq] * kLog2e;
      negd = -part[0];
    }
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = df[s] = u32x4{0, 0, 0, 0};
  }
  if (!GEN && a.rowterm_here && qw < N && hh == 0) {   // (rows past N of the block: zeros)
    const long long t = rowterm_index((long long)b * a.Hq + hq, (N + 31) / 32, myq);
    a.rowterm[t] = lse2;
    a.rowterm[t + 32] = negd;
  }
  // dP^T of every unit starts from -D (this lane's query), so dP - D comes out of the MFMA
  f32x16 ndv;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndv[i] = negd;

  const int nkv = (Lk + BC - 1) / BC;
  // Key tiles visited, in order: tile_of(j), j < ntile (the mask family: the tiles of the
  // workgroup's key interval, filtered by its 256-query block's list when there is one);
  // masked head [0, JH), plain [JH, JT), masked tail [JT, ntile) (a tile's flag covers
  // its own two units)
  int ntile, t_lo = 0, p0 = 0, JH = 0, JT = 0;
  const int* lst = nullptr;
  int lo_q = 0, hi_q = Lk - 1, wlo = 0, whi;
  if constexpr (GEN) {
    const int qlast = min(q0 + BR, Lq) - 1;
    auto lo_of = [&](int i) { return a.wl >= 0 ? i + off - a.wl : 0; };
    auto hi_of = [&](int i) { return a.wr >= 0 ? min(i + off + a.wr, Lk - 1) : Lk - 1; };
    lo_q = lo_of(myq);
    hi_q = hi_of(myq);
    wlo = max(lo_of(min(qw + 31, Lq - 1)), 0);
    whi = hi_of(qw);
    const int klo = max(lo_of(q0), 0), khi = hi_of(qlast);
    t_lo = klo / BC;
    const int t_hi = (Lk <= 0 || khi < klo) ? t_lo : khi / BC + 1;
    // tiles that need element masks: below the largest lower bound, or past the smallest
    // upper bound (which includes the tile holding key Lk-1 when Lk is ragged)
    const int tm_head = (max(lo_of(qlast), 0) + BC - 1) / BC;
    const int tm_tail = (hi_of(q0) + 1) / BC;
    int P1, P2;
    if (a.bidx != nullptr) {
      static_assert(256 % BR == 0, "a workgroup's queries lie in one 256-query block of the lists");
      const int hm = a.bheads == 1 ? 0 : hq;
      const size_t row = ((size_t)b * a.bheads + hm) * a.bnq + q0 / 256;
      const int cnt = min(max(a.bcnt[row], 0), a.bcap);
      lst = a.bidx + row * a.bcap;
      p0 = lower_bound_tiles(lst, cnt, t_lo);
      ntile = lower_bound_tiles(lst, cnt, t_hi) - p0;
      P1 = lower_bound_tiles(lst, cnt, tm_head) - p0;
      P2 = lower_bound_tiles(lst, cnt, tm_tail) - p0;
    } else {
      ntile = t_hi - t_lo;
      P1 = tm_head - t_lo;
      P2 = tm_tail - t_lo;
    }
    P1 = min(max(P1, 0), ntile);
    P2 = min(max(P2, 0), ntile);
    JH = min(ntile, (P1 + NSL - 1) / NSL * NSL);
    JT = max(JH, P2 / NSL * NSL);
  } else {
    ntile = CAUSAL ? min(nkv, (min(q0 + BR, N) - 1) / BC + 1) : nkv;
    whi = CAUSAL ? min(qw, N - 1) : N - 1;
  }
  // tile index of list position j
  auto tile_of = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (!GEN) return j;
    if (lst == nullptr) return t_lo + j;
    return min(max(lst[p0 + j], t_lo), nkv - 1);
  };
  // keys some query of this wave sees: [ulo, uhi] (empty when the wave has no query)
  int ulo = 0, uhi;
  if constexpr (GEN) {
    ulo = max(a.wl >= 0 ? qw + off - a.wl : 0, 0);
    uhi = qw >= Lq ? -1 : a.wr >= 0 ? min(min(qw + 31, Lq - 1) + off + a.wr, Lk - 1) : Lk - 1;
  } else {
    uhi = qw >= N ? -1 : CAUSAL ? min(qw + 31, N - 1) : N - 1;
  }

  int doff[IPW];
  Tiles::offsets(wave, lane, doff);
  auto dma = [&](int t, unsigned char* sl) __attribute__((always_inline)) {
    Tiles::load(Kg, Vg, Lk, tile_of(t), wave, doff, sl);
  };

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
  const int va = r32 * PV + 16 * hh;

  const float c2 = a.scale_log2;
  f32x16 acc[NE];
  acc_init(acc);

  // unit = 32 keys: half h of the tile in slot sl
  auto krow = [&](const unsigned char* sl, int h, int st) __attribute__((always_inline)) {
    return *(const u32x4*)(sl + h * 32 * PK + ka[st]);
  };
  auto vrow = [&](const unsigned char* sl, int h, int st) __attribute__((always_inline)) {
    return *(const u32x4*)(sl + KBYTES + h * 32 * PV + va + 32 * st);
  };
  auto ktr = [&](const unsigned char* sl, int h, int t, int e) __attribute__((always_inline)) {
    return cat(lds_read_tr(sl + (32 * h + 16 * t) * PK + kt[2 * e]),
               lds_read_tr(sl + (32 * h + 16 * t + 8) * PK + kt[2 * e + 1]));
  };
  // dS of one unit from its S^T and dP^T - D
  auto dsfrom = [&](f32x16& s, const f32x16& dp, int lo, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (v >= lo && v < hi) {
        const float p = fast_exp2(fmaf(s[v], c2, -lse2));
        s[v] = p * dp[v];
        keep(s[v]);
      }
  };
  auto pack = [&](const f32x16& s, int h) __attribute__((always_inline)) {
    return u32x4{E::pack(s[8 * h + 0], s[8 * h + 1]), E::pack(s[8 * h + 2], s[8 * h + 3]),
                 E::pack(s[8 * h + 4], s[8 * h + 5]), E::pack(s[8 * h + 6], s[8 * h + 7])};
  };
  auto accumulate = [&](const unsigned char* sl, int h, const u32x4* pf) __attribute__((always_inline)) {
    u32x4 tf = ktr(sl, h, 0, 0);
#pragma unroll
    for (int k = 0; k < 2 * NE; ++k) {
      const int t = k / NE, e = k % NE;
      const u32x4 cur = tf;
      if (k + 1 < 2 * NE) tf = ktr(sl, h, (k + 1) / NE, (k + 1) % NE);
      if (k == 0) A::mma_fresh(acc[e], cur, pf[t]);
      else A::mma(acc[e], cur, pf[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Unit u in (sc, dpc) from half hc of slot slc; the next unit's products (half hn of
  // slot sln) are formed into (sn, dpn) interleaved with this unit's elementwise dS, then
  // dQ^T += K_u^T dS_u^T.  MASK: zero dS where the key is past N or (causal) after the
  // query; a unit wholly past the wave's last one then adds zeros.
  auto step = [&](auto MASK, int u, const unsigned char* slc, int hc, const unsigned char* sln, int hn,
                  f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn) __attribute__((always_inline)) {
    u32x4 kf = krow(sln, hn, 0), vf = vrow(sln, hn, 0);
    u32x4 pf[2];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const u32x4 kc = kf, vc = vf;
      if (k + 1 < NS) {
        kf = krow(sln, hn, k + 1);
        vf = vrow(sln, hn, k + 1);
      }
      dsfrom(sc, dpc, (16 * k) / NS, (16 * (k + 1)) / NS);
      sn = E::mma(kc, qf[k], k == 0 ? zero16() : sn);
      dpn = E::mma(vc, df[k], k == 0 ? ndv : dpn);
      if (k == NS - 1) {
        if constexpr (decltype(MASK)::value) {
          // keys k0 + 8(v/4) + 4hh + v%4 of this lane's column; a unit every query of the
          // wave sees whole needs nothing
          const int k0 = GEN ? tile_of(u >> 1) * BC + 32 * (u & 1) : u * 32;
          if (!(k0 >= wlo && k0 + 31 <= whi)) {
            int lim = (GEN ? min(Lk, hi_q + 1) : N) - k0 - 4 * hh;
            if (!GEN && CAUSAL) lim = min(lim, myq - k0 - 4 * hh + 1);
            const int llo = lo_q - k0 - 4 * hh;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int o = 8 * (v >> 2) + (v & 3);
              if (o >= lim || (GEN && o < llo)) sc[v] = 0.f;
            }
          }
        }
        pf[0] = pack(sc, 0);
        pf[1] = pack(sc, 1);
        keep(pf[0]);
        keep(pf[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    accumulate(slc, hc, pf);
  };

  // Without PIPE: unit u's S^T, dP^T from half h of slot sl, then its dS (masked as in
  // step) and dQ^T += K_u^T dS_u^T; in masked tiles a unit the wave cannot see is skipped.
  auto step1 = [&](auto MASK, int u, const unsigned char* sl, int h) __attribute__((always_inline)) {
    if constexpr (decltype(MASK)::value) {
      // a unit no query of this wave sees adds nothing: skip it (wave-uniform; the other
      // wave on the SIMD takes the freed cycles)
      const int k0 = GEN ? tile_of(u >> 1) * BC + 32 * (u & 1) : u * 32;
      if (k0 > uhi || k0 + 31 < ulo) return;
    }
    u32x4 kf = krow(sl, h, 0), vf = vrow(sl, h, 0);
    f32x16 s, dp;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const u32x4 kc = kf, vc = vf;
      if (k + 1 < NS) {
        kf = krow(sl, h, k + 1);
        vf = vrow(sl, h, k + 1);
      }
      s = E::mma(kc, qf[k], k == 0 ? zero16() : s);
      dp = E::mma(vc, df[k], k == 0 ? ndv : dp);
    }
    dsfrom(s, dp, 0, 16);
    if constexpr (decltype(MASK)::value) {
      const int k0 = GEN ? tile_of(u >> 1) * BC + 32 * (u & 1) : u * 32;
      if (!(k0 >= wlo && k0 + 31 <= whi)) {
        int lim = (GEN ? min(Lk, hi_q + 1) : N) - k0 - 4 * hh;
        if (!GEN && CAUSAL) lim = min(lim, myq - k0 - 4 * hh + 1);
        const int llo = lo_q - k0 - 4 * hh;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int o = 8 * (v >> 2) + (v & 3);
          if (o >= lim || (GEN && o < llo)) s[v] = 0.f;
        }
      }
    }
    const u32x4 pf[2] = {pack(s, 0), pack(s, 1)};
    accumulate(sl, h, pf);
  };

  f32x16 sa, pa, sb, pb;
  // Tile j (slot T = j % NSL): sync, load tile j + NSL - 1 into the slot tile j-1 used,
  // units 2j (S, dP in sa, pa) and 2j+1 (in sb, pb).  With PIPE, the products of the
  // unit after the last are formed from a valid slot and never used.
  auto tile = [&](auto Tc, auto MASK, int j) __attribute__((always_inline)) {
    constexpr int T = decltype(Tc)::value;
    unsigned char* const sc = slot(T);
    unsigned char* const sn = slot((T + 1) % NSL);
    if (j > 0) {
      wait_loads();      // this wave's loads of tiles up to j + 1 (NSL = 3), j (NSL = 2)
      __syncthreads();   // everyone's; everyone is done with tile j-1
    }
    if (j + NSL - 1 < ntile) dma(j + NSL - 1, slot((T + NSL - 1) % NSL));
    if constexpr (PIPE) {
      step(MASK, 2 * j, sc, 0, sc, 1, sa, pa, sb, pb);
      step(MASK, 2 * j + 1, sc, 1, sn, 0, sb, pb, sa, pa);
    } else {
      step1(MASK, 2 * j, sc, 0);
      step1(MASK, 2 * j + 1, sc, 1);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using Plain = std::false_type;
  using Masked = std::true_type;

  if (!GEN || ntile > 0) {   // (a mask-family workgroup may have no key tile)
  dma(0, slot0);
  if (NSL == 3 && ntile > 1) dma(1, slot1);
  wait_loads();
  __syncthreads();
  if constexpr (PIPE) {
    sa = zero16();
    pa = ndv;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      sa = E::mma(krow(slot0, 0, st), qf[st], sa);
      pa = E::mma(vrow(slot0, 0, st), df[st], pa);
    }
  }
  // Tiles whose units all precede every wave's last unit need no mask.
  if constexpr (!GEN) {
    const int ulast0 = (CAUSAL ? min(q0 + 31, N - 1) : N - 1) / 32;
    JT = min(ntile, ulast0 / 2) / NSL * NSL;
  }
  int j = 0;
  for (; j < JH; j += NSL) {
    tile(I0{}, Masked{}, j);
    if (j + 1 >= ntile) break;
    tile(I1{}, Masked{}, j + 1);
    if constexpr (NSL == 3) {
      if (j + 2 >= ntile) break;
      tile(I2{}, Masked{}, j + 2);
    }
  }
  j = JH;
  for (; j < JT; j += NSL) {
    tile(I0{}, Plain{}, j);
    tile(I1{}, Plain{}, j + 1);
    if constexpr (NSL == 3) tile(I2{}, Plain{}, j + 2);
  }
  for (; j < ntile; j += NSL) {
    tile(I0{}, Masked{}, j);
    if (j + 1 >= ntile) break;
    tile(I1{}, Masked{}, j + 1);
    if constexpr (NSL == 3) {
      if (j + 2 >= ntile) break;
      tile(I2{}, Masked{}, j + 2);
    }
  }
  }
  acc_drain(acc);

  // dQ = scale * (dQ^T)^T, rounded to the input dtype
  if (myq < Lq) {
    store_row16<E>((unsigned char*)a.dq + (qhead + myq) * ROWB, acc, a.scale, hh);
  }
}

// Waves per workgroup of the dQ pass (two waves per SIMD either way): 8 (256 queries,
// one workgroup per CU) or 4 (two per CU).  d = 64: 4 (51 KB of LDS each; measured as
// fast or faster at every shape).  d = 128: 4 while the 256-row grid is small — at most
// 128 workgroups, or 256 when causal — where it would leave CUs idle, and under a
// window whose left side is shorter than 2048 keys, where a workgroup's key span
// (window + its rows) exceeds each wave's (window + 32) by a large fraction and the
// narrower workgroup wastes less; elsewhere the two workgroups' separate K/V streams
// cost 1-3 %.
template <int D>
static int dq_waves(long long blocks_of_256, bool causal, int window_left) {
  if (D != 128) return 4;
  if (window_left >= 0 && window_left < 2048) return 4;
  return blocks_of_256 <= (causal ? 256 : 128) ? 4 : 8;
}

template <class Tag, int D, bool CAUSAL, bool GEN>
static hipError_t launch_dq(const BwdArgs& a, int nq, bool causal, hipStream_t stream) {
  const long long bh = (long long)a.B * a.Hq;
  constexpr bool PIPE = D != 128;   // d = 128: one unit at a time (see the dQ pass)
  if (dq_waves<D>(bh * ((nq + 255) / 256), causal, GEN ? a.wl : -1) == 4) {
    const long long nb = bh * ((nq + 127) / 128);
    hipLaunchKernelGGL((bwd_dq_kernel<Tag, D, CAUSAL, 4, PIPE, GEN>), dim3((unsigned)nb), dim3(4 * 64), 0, stream, a);
  } else {
    const long long nb = bh * ((nq + 255) / 256);
    hipLaunchKernelGGL((bwd_dq_kernel<Tag, D, CAUSAL, 8, PIPE, GEN>), dim3((unsigned)nb), dim3(8 * 64), 0, stream, a);
  }
  return hipGetLastError();
}

template <class Tag, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a0, hipStream_t stream) {
  const long long prows = (long long)a0.B * a0.Hq * ((a0.N + 31) / 32) * 32;   // padded rows
  if (prows <= 0) return hipSuccess;
  BwdArgs a = a0;
  a.rowterm_here = 1;   // the dQ pass forms and writes the row terms (no row-term kernel)
  hipError_t err = launch_dq<Tag, D, CAUSAL, false>(a, a.N, CAUSAL, stream);
  if (err != hipSuccess) return err;
  if (a.kblock == 256) {   // 64 keys a wave
    const long long nrec256 = (a.N + 255) / 256 * a.B * a.Hkv;
    if (a.ksplit == 1) {
      hipLaunchKernelGGL((bwd_dkdv64_kernel<Tag, D, CAUSAL>), dim3((unsigned)nrec256), dim3(256), 0, stream, a);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((bwd_dkdv64_kernel<Tag, D, CAUSAL, true>), dim3((unsigned)(nrec256 * a.ksplit)), dim3(256), 0,
                       stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((bwd_reduce_kernel<Tag, D>), dim3((unsigned)(nrec256 * a.ksplit)), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const long long nrec = (a.N + 127) / 128 * a.B * a.Hkv;
  if (a.ksplit == 1) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<Tag, D, CAUSAL>), dim3((unsigned)nrec), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bwd_dkdv_kernel<Tag, D, CAUSAL, false, true>), dim3((unsigned)(nrec * a.ksplit)), dim3(256), 0,
                     stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((bwd_reduce_kernel<Tag, D>), dim3((unsigned)(nrec * a.ksplit)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class Tag, int D>
static hipError_t launch_bwd_masked_t(const BwdArgs& a, hipStream_t stream) {
  const long long prows = (long long)a.B * a.Hq * ((a.maxq + 31) / 32) * 32;   // padded rows
  if (prows <= 0) return hipSuccess;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_rowterm_kernel<Tag, D, true>), dim3((unsigned)((prows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, a, prows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_dq<Tag, D, false, true>(a, a.maxq, a.wr >= 0, stream);
  if (err != hipSuccess) return err;
  const long long nkb = (a.maxk + 127) / 128;
  if (nkb <= 0) return hipSuccess;
  const long long nrec = (long long)a.B * a.Hkv * nkb;
  if (a.runs != nullptr) {
    hipLaunchKernelGGL(bwd_runs_kernel, dim3((unsigned)((nrec + 3) / 4)), dim3(256), 0, stream, a, nrec, (int)nkb);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(1024), 0, stream, a, (int)nrec);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const long long extra = a.runs != nullptr ? kBwdSlots : 0;   // later chunks of split key blocks, first
  hipLaunchKernelGGL((bwd_dkdv_kernel<Tag, D, false, true>), dim3((unsigned)(nrec + extra)), dim3(256), 0, stream,
                     a);
  err = hipGetLastError();
  if (err != hipSuccess || a.runs == nullptr) return err;
  hipLaunchKernelGGL((bwd_reduce_kernel<Tag, D>), dim3(kBwdSlots), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_masked(const BwdArgs& a, int d, bool bf16, hipStream_t stream) {
  if (bf16) return d == 128 ? launch_bwd_masked_t<bf16_tag, 128>(a, stream) : launch_bwd_masked_t<bf16_tag, 64>(a, stream);
  return d == 128 ? launch_bwd_masked_t<f16_tag, 128>(a, stream) : launch_bwd_masked_t<f16_tag, 64>(a, stream);
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
