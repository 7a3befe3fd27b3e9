// Split-KV forward for decoding (few queries, long key/value sequence) and the
// log-sum-exp combine of partial results, for gfx950.
//
// Method: "Flash Attention" (wiki), section "Training and autoregressive decoding"
// (one new query against a long cache leaves too few query blocks to fill the GPU)
// and section "Flash-Decoding": the key/value sequence is split into chunks, each
// chunk is attended with the FlashAttention recurrence, and the partial outputs are
// merged with their log-sum-exp statistics in a small reduction.  Queries are the
// last Nq positions of the sequence (query i at position Nk - Nq + i; causal: keys
// j <= Nk - Nq + i).
//
// gfx950 design.
//  * Decoding is bound by HBM bandwidth: every K/V byte is read once per split and
//    the arithmetic is small.  The work unit is therefore a split, and a split is
//    one wave: a workgroup is four independent waves (four splits), with no barrier.
//  * A wave owns the 32 query rows of one (batch, K/V head) group: the G = Hq/Hkv
//    query heads times Nq queries, lane % 32 = row (rows past G*Nq are zero padding;
//    more rows run as further row groups).  Scores are formed transposed as in the
//    forward kernel, S^T = K Q^T, so the softmax is per lane and P is already the B
//    operand of O^T += V^T P^T.
//  * K feeds the MFMA A operand straight from HBM (each lane reads 16 contiguous bytes
//    of one key row).  V needs a transposed operand, so it goes HBM -> LDS with
//    buffer loads into the wave's own slot (rows padded to row+64 bytes) and is read
//    back with ds_read_b64_tr_b16.  Both are issued two 32-key units ahead; a wave
//    waits only for its own loads (s_waitcnt vmcnt), never for other waves.
//  * The three V slots are distinct LDS objects indexed at compile time (the unit
//    loop is unrolled by 3), so the compiler does not make the transposing reads of
//    one slot wait for the loads into another.
//  * The four splits of a workgroup merge their partial results in LDS; the workgroup
//    writes one normalised partial O (fp32) and partial LSE per row, and the combine
//    kernel merges those per row.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// s_waitcnt vmcnt(N) (the other counters untouched)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((((N >> 4) & 3) << 14) | (0xF << 8) | (0x7 << 4) | (N & 15));
}

// One 32-key V tile (rows of ROWB bytes, padded to pitch PV in LDS) of the unit whose
// first key is at byte kb_bytes of the head, into this wave's slot `dst`.  Load i
// covers slot bytes [1024i, 1024i + 1024); lanes landing on row padding fetch any
// in-range byte.  The descriptor's range ends at the head's last key, so keys past
// it arrive as zeros.  (A free function: the host pass of the compiler mishandles
// these builtins inside a capturing lambda.)
template <int ROWB, int NLOAD>
__device__ __forceinline__ void vtile_dma(const unsigned char* vhead, int head_bytes, int kb_bytes, const int* voff,
                                          unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)vhead, (short)0, head_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < NLOAD; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lvoid*)(dst + i * 1024), 16, voff[i] + kb_bytes, 0, 0, 0);
}

// The K fragments of one 32-key unit as MFMA A operands: lane holds key kb + lane%32,
// elements 16st + 8(lane/32) .. +7.  Keys past the head's end read as zeros.
template <int ROWB, int NS>
__device__ __forceinline__ void ktile_load(const unsigned char* khead, int head_bytes, int voff, u32x4* kf) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)khead, (short)0, head_bytes, 0x00020000);
#pragma unroll
  for (int st = 0; st < NS; ++st)
    kf[st] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 32 * st, 0, 0));
}

template <class Tag, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) splitkv_kernel(const DecodeArgs a) {
  using E = Elt<Tag>;
  constexpr int NW = 4;
  constexpr int ROWB = D * 2;
  constexpr int NS = D / 16;            // k-steps of S^T
  constexpr int NE = D / 32;            // 32-row blocks of O^T
  constexpr int PV = ROWB + 64;         // LDS pitch of V rows (transposing reads)
  constexpr int VBYTES = 32 * PV;       // one 32-key V tile
  constexpr int NLOAD = VBYTES / 1024;  // wave-wide 16-byte loads per V tile
  constexpr int PER = NLOAD + NS;       // vector-memory instructions per unit
  constexpr float TAU = 8.f;            // rescale threshold (log2 units)
  static_assert(VBYTES % 1024 == 0, "V tile is whole wave loads");

  __shared__ __attribute__((aligned(1024))) unsigned char vs0[NW * VBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vs1[NW * VBYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vs2[NW * VBYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int Nq = a.Nq, Nk = a.Nk;
  const int G = a.Hq / a.Hkv;

  // block -> (group, split quad, row group); row groups innermost so that the blocks
  // reading the same K/V chunk run together
  int bid = blockIdx.x;
  const int rg = bid % a.RG;
  bid /= a.RG;
  const int nquad = a.S4 / NW;
  const int quad = bid % nquad;
  const int grp = bid / nquad;
  const int b = grp / a.Hkv, hkv = grp - b * a.Hkv;
  const int s = quad * NW + wave;                     // this wave's split
  const int ks = s * a.C;
  const int ke = min(ks + a.C, Nk);

  const int r = rg * 32 + r32;                        // row of the group
  const bool valid = r < G * Nq;
  const int g = valid ? r / Nq : 0;
  const int qi = valid ? r - g * Nq : 0;
  const int hq = hkv * G + g;
  const int qpos = Nk - Nq + qi;                      // absolute position of the query
  const long long orow = ((long long)(b * a.Hq + hq)) * Nq + qi;

  const int nunit = ks < ke ? (ke - ks + 31) / 32 : 0;   // 0: an empty split (past the keys)

  // Q^T as the B operand: lane holds Q[row][16st + 8hh .. +7]
  u32x4 qf[NS];
  if (valid) {
    const unsigned char* qp = (const unsigned char*)a.q + orow * ROWB + 16 * hh;
#pragma unroll
    for (int st = 0; st < NS; ++st) qf[st] = *(const u32x4*)(qp + 32 * st);
  } else {
#pragma unroll
    for (int st = 0; st < NS; ++st) qf[st] = u32x4{0, 0, 0, 0};
  }

  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)Nk * ROWB;
  const unsigned char* Kh = (const unsigned char*)a.k + kvhead;
  const unsigned char* Vh = (const unsigned char*)a.v + kvhead;
  const int head_bytes = Nk * ROWB;
  int voff[NLOAD];
#pragma unroll
  for (int i = 0; i < NLOAD; ++i) {
    const int o = i * 1024 + lane * 16;
    const int row = o / PV, col = o - (o / PV) * PV;
    voff[i] = row * ROWB + (col < ROWB ? col : 0);
  }
  const int koff = r32 * ROWB + 16 * hh;
  // V (A operand of O^T, read transposed): row 16t + 8u + R, element 32e + 16x + 4y
  const int va = wave * VBYTES + (4 * hh + ((lane & 15) >> 2)) * PV + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  auto vread = [&](const unsigned char* sl, int h, int e) __attribute__((always_inline)) {
    const unsigned char* p = sl + va;
    return cat(lds_read_tr(p + 16 * h * PV + 64 * e), lds_read_tr(p + (16 * h + 8) * PV + 64 * e));
  };
  auto issue = [&](int u, u32x4* kf, unsigned char* sl) __attribute__((always_inline)) {
    const int kb = ks + 32 * u;
    vtile_dma<ROWB, NLOAD>(Vh, head_bytes, kb * ROWB, voff, sl + wave * VBYTES);
    ktile_load<ROWB, NS>(Kh, head_bytes, kb * ROWB + koff, kf);
  };

  const float c2 = a.scale_log2;
  float mr = -INFINITY, l_run = 0.f;
  f32x16 o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e] = zero16();

  // unit u: S^T = K Q^T, mask, online softmax (reference raised past TAU), O^T += V^T P^T
  auto compute = [&](int u, const u32x4* kf, const unsigned char* sl) __attribute__((always_inline)) {
    const int kb = ks + 32 * u;
    f32x16 sc = zero16();
#pragma unroll
    for (int st = 0; st < NS; ++st) sc = E::mma(kf[st], qf[st], sc);
    if (kb + 32 > ke || (CAUSAL && kb + 31 > Nk - Nq)) {
      // keys kb + 8(v/4) + 4hh + v%4 of this lane's column
      int lim = ke - kb - 4 * hh;
      if (CAUSAL) lim = min(lim, qpos + 1 - kb - 4 * hh);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + (v & 3) >= lim) sc[v] = -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    mx = half_max(mx) * c2;
    const bool raise = mx > mr + TAU;
    const float mnew = raise ? mx : mr;
    const float alpha = (mr == -INFINITY) ? 0.f : fast_exp2(mr - mnew);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    mr = mnew;
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sc[v] = fast_exp2(fmaf(sc[v], c2, -mref));
      rs += sc[v];
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[e][v] *= alpha;
    }
    const u32x4 pf[2] = {
        u32x4{E::pack(sc[0], sc[1]), E::pack(sc[2], sc[3]), E::pack(sc[4], sc[5]), E::pack(sc[6], sc[7])},
        u32x4{E::pack(sc[8], sc[9]), E::pack(sc[10], sc[11]), E::pack(sc[12], sc[13]), E::pack(sc[14], sc[15])}};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < NE; ++e) o[e] = E::mma(vread(sl, h, e), pf[h], o[e]);
    l_run = fmaf(l_run, alpha, rs);
  };

  // unit u (slot J % 3): issue unit u+2, wait for unit u's loads, compute unit u
  auto step = [&](auto Jc, int u, const u32x4* kcur, u32x4* kpf) __attribute__((always_inline)) {
    constexpr int J = decltype(Jc)::value;
    unsigned char* const cur = J == 0 ? vs0 : J == 1 ? vs1 : vs2;
    unsigned char* const pf = J == 0 ? vs2 : J == 1 ? vs0 : vs1;
    if (u + 2 < nunit) {
      issue(u + 2, kpf, pf);
      wait_vm<2 * PER>();
    } else if (u + 1 < nunit) {
      wait_vm<PER>();
    } else {
      wait_vm<0>();
    }
    compute(u, kcur, cur);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  u32x4 kA[NS], kB[NS], kC[NS];
  if (nunit > 0) issue(0, kA, vs0);
  if (nunit > 1) issue(1, kB, vs1);
  for (int u = 0; u < nunit; u += 3) {
    step(I0{}, u, kA, kC);
    if (u + 1 >= nunit) break;
    step(I1{}, u + 1, kB, kA);
    if (u + 2 >= nunit) break;
    step(I2{}, u + 2, kC, kB);
  }

  // Partial result of this split (O normalised over its keys, LSE in natural log),
  // merged in LDS with the other three splits of the workgroup by the combine rule; the
  // workgroup writes one part per row.  The V slots are reused once every wave is done.
  const float l_tot = half_sum(l_run);
  const float lse_w = l_tot > 0.f ? (mr + log2f(l_tot)) * kLn2 : -INFINITY;
  __syncthreads();
  float* po = (float*)(wave < 2 ? vs0 : vs1) + (wave & 1) * 32 * D;   // [32 rows][D] of this wave
  float* pl = (float*)vs2 + wave * 32;                               // [32 rows]
  {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * e + 8 * g4 + 4 * hh;
        const f32x4 w = {o[e][4 * g4 + 0] * inv, o[e][4 * g4 + 1] * inv, o[e][4 * g4 + 2] * inv,
                         o[e][4 * g4 + 3] * inv};
        *(f32x4*)(po + r32 * D + d0) = w;
      }
    if (hh == 0) pl[r32] = lse_w;
  }
  __syncthreads();
  // thread t: row t / 8, elements (t % 8) * D/8 .. +D/8
  {
    constexpr int EPT = D / 8;
    const int t = threadIdx.x, row = t >> 3, e0 = (t & 7) * EPT;
    const int rr = rg * 32 + row;
    if (rr < G * Nq) {
      const int rg_g = rr / Nq, rq = rr - rg_g * Nq;
      const long long orr = ((long long)(b * a.Hq + hkv * G + rg_g)) * Nq + rq;
      float lw[NW], M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        lw[w] = ((const float*)vs2)[w * 32 + row];
        M = fmaxf(M, lw[w]);
      }
      float wt[NW], den = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        wt[w] = (M == -INFINITY || lw[w] == -INFINITY) ? 0.f : fast_exp2((lw[w] - M) * kLog2e);
        den += wt[w];
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const int P = a.S4 / NW;                        // parts per row: one per workgroup
      float* dst = a.opart + (orr * P + quad) * D + e0;
#pragma unroll
      for (int i = 0; i < EPT; i += 4) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          if (wt[w] == 0.f) continue;
          const float* src = (const float*)(w < 2 ? vs0 : vs1) + (w & 1) * 32 * D + row * D + e0 + i;
          const f32x4 x = *(const f32x4*)src;
          acc += wt[w] * x;
        }
        *(f32x4*)(dst + i) = acc * inv;
      }
      if ((t & 7) == 0) a.lpart[orr * P + quad] = den > 0.f ? M + logf(den) : -INFINITY;
    }
  }
}

// ---- combine: per row, O = sum_s w_s O_s / sum_s w_s, LSE = M + ln sum_s w_s,
// w_s = exp(LSE_s - M), M = max_s LSE_s; parts with LSE_s = -inf carry no weight.
// One 256-thread workgroup per row: 256/D groups of D threads each take every
// (256/D)-th part, loading a chunk of parts at once (one memory round trip per chunk)
// and merging chunks with a running maximum; the groups are merged in LDS.
template <class Tag, int D>
__global__ void __launch_bounds__(256) lse_combine_kernel(const float* opart, const float* lpart, void* o, float* lse,
                                                          long long rows, int S) {
  using E = Elt<Tag>;
  constexpr int NT = 256;
  constexpr int NG = NT / D;            // thread groups over the parts
  constexpr int CH = 16;                // parts per thread per chunk
  __shared__ float gm[NG], gden[NG];
  __shared__ float gacc[NG][D];
  const long long row = (long long)blockIdx.y * gridDim.x + blockIdx.x;
  if (row >= rows) return;              // uniform per workgroup
  const int t = threadIdx.x;
  const int g = t / D, e = t - (t / D) * D;
  const float* lp = lpart + row * S;
  const float* op = opart + row * (long long)S * D + e;
  float m = -INFINITY, den = 0.f, acc = 0.f;
  for (int base = g; base < S; base += NG * CH) {
    float lv[CH], ov[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int si = base + i * NG;
      lv[i] = si < S ? lp[si] : -INFINITY;
      ov[i] = si < S ? op[(long long)si * D] : 0.f;
    }
    float cm = lv[0];
#pragma unroll
    for (int i = 1; i < CH; ++i) cm = fmaxf(cm, lv[i]);
    const float nm = fmaxf(m, cm);
    if (nm == -INFINITY) continue;
    const float sc = m == -INFINITY ? 0.f : fast_exp2((m - nm) * kLog2e);
    den *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (lv[i] == -INFINITY) continue;           // empty part: its O was never written
      const float w = fast_exp2((lv[i] - nm) * kLog2e);
      den += w;
      acc = fmaf(w, ov[i], acc);
    }
    m = nm;
  }
  if (e == 0) {
    gm[g] = m;
    gden[g] = den;
  }
  gacc[g][e] = acc;
  __syncthreads();
  if (t < D) {
    float M = gm[0];
#pragma unroll
    for (int i = 1; i < NG; ++i) M = fmaxf(M, gm[i]);
    float dd = 0.f, aa = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        if (gm[i] == -INFINITY) continue;
        const float w = fast_exp2((gm[i] - M) * kLog2e);
        dd += w * gden[i];
        aa += w * gacc[i][t];
      }
    }
    const float inv = dd > 0.f ? 1.f / dd : 0.f;
    const float nb = __shfl_down(aa, 1, 64);
    if ((t & 1) == 0) *(uint32_t*)((unsigned char*)o + row * (D * 2) + t * 2) = E::pack(aa * inv, nb * inv);
    if (t == 0) lse[row] = dd > 0.f ? M + logf(dd) : -INFINITY;
  }
}

// The same combine for few parts (S <= 16) and many rows: D/4 threads per row, four
// adjacent elements each (one 16-byte load per part), 256 / (D/4) rows per workgroup.
// Every thread of a row reads the row's S statistics (the same cache lines).
template <class Tag, int D>
__global__ void __launch_bounds__(256) lse_combine_rows_kernel(const float* opart, const float* lpart, void* o,
                                                               float* lse, long long rows, int S) {
  using E = Elt<Tag>;
  constexpr int TPR = D / 4;             // threads per row
  const long long row = ((long long)blockIdx.y * gridDim.x + blockIdx.x) * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int e4 = (threadIdx.x % TPR) * 4;
  const float* lp = lpart + row * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[s]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    const float* op = opart + row * (long long)S * D + e4;
    for (int s = 0; s < S; ++s) {
      const float l = lp[s];
      if (l == -INFINITY) continue;              // empty part: its O carries no weight
      const float w = fast_exp2((l - M) * kLog2e);
      den += w;
      acc += w * *(const f32x4*)(op + (long long)s * D);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const u32x2 w = {E::pack(acc[0] * inv, acc[1] * inv), E::pack(acc[2] * inv, acc[3] * inv)};
  *(u32x2*)((unsigned char*)o + row * (D * 2) + e4 * 2) = w;
  if (e4 == 0) lse[row] = den > 0.f ? M + logf(den) : -INFINITY;
}

template <class Tag, int D>
static hipError_t launch_combine_t(const float* opart, const float* lpart, void* o, float* lse, long long rows, int S,
                                   hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (S <= 16) {
    const long long nb = (rows + 256 / (D / 4) - 1) / (256 / (D / 4));
    const unsigned gx = (unsigned)(nb < 65536 ? nb : 65536);
    const unsigned gy = (unsigned)((nb + gx - 1) / gx);
    hipLaunchKernelGGL((lse_combine_rows_kernel<Tag, D>), dim3(gx, gy), dim3(256), 0, stream, opart, lpart, o, lse,
                       rows, S);
    return hipGetLastError();
  }
  const unsigned gx = (unsigned)(rows < 65536 ? rows : 65536);
  const unsigned gy = (unsigned)((rows + gx - 1) / gx);
  hipLaunchKernelGGL((lse_combine_kernel<Tag, D>), dim3(gx, gy), dim3(256), 0, stream, opart, lpart, o, lse, rows, S);
  return hipGetLastError();
}

template <class Tag, int D, bool CAUSAL>
static hipError_t launch_splitkv_t(const DecodeArgs& a, hipStream_t stream) {
  const long long nblocks = (long long)a.B * a.Hkv * a.RG * (a.S4 / 4);
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((splitkv_kernel<Tag, D, CAUSAL>), dim3((unsigned)nblocks), dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine_t<Tag, D>(a.opart, a.lpart, a.o, a.lse, (long long)a.B * a.Hq * a.Nq, a.S4 / 4, stream);
}

hipError_t launch_splitkv(const DecodeArgs& a, int d, bool bf16, bool causal, hipStream_t stream) {
#define FA_DEC_CASE(TAG, D) \
  return causal ? launch_splitkv_t<TAG, D, true>(a, stream) : launch_splitkv_t<TAG, D, false>(a, stream)
  if (bf16) {
    if (d == 128) FA_DEC_CASE(bf16_tag, 128);
    FA_DEC_CASE(bf16_tag, 64);
  } else {
    if (d == 128) FA_DEC_CASE(f16_tag, 128);
    FA_DEC_CASE(f16_tag, 64);
  }
#undef FA_DEC_CASE
}

hipError_t launch_lse_combine(const float* opart, const float* lpart, void* o, float* lse, long long rows, int S,
                              int d, bool bf16, hipStream_t stream) {
  if (bf16) return d == 128 ? launch_combine_t<bf16_tag, 128>(opart, lpart, o, lse, rows, S, stream)
                            : launch_combine_t<bf16_tag, 64>(opart, lpart, o, lse, rows, S, stream);
  return d == 128 ? launch_combine_t<f16_tag, 128>(opart, lpart, o, lse, rows, S, stream)
                  : launch_combine_t<f16_tag, 64>(opart, lpart, o, lse, rows, S, stream);
}

}  // namespace fa
