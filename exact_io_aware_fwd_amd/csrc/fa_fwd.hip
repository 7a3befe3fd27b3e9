// Forward pass of exact attention for gfx950: tiled, online softmax, O and LSE only.
//
// Method: "FlashAttention Primer: IO-Aware Attention, from FA1 to FA4", section
// "FlashAttention-1: tiling plus online softmax" (Figures 3 and 4): Q row blocks
// outer, K/V column blocks inner, running max m, running sum l and unnormalised
// output kept on chip, one division at the end; causal tiles above the diagonal
// are skipped.  Work split as in the section "FlashAttention-2: better work
// partitioning" (Figure 6): one workgroup per (batch, head, query block), so no
// atomics and a bitwise-deterministic result.  The rescaling threshold follows
// the section "FlashAttention-4: Blackwell co-design" (conditional softmax
// rescaling); the overlap of score products with the softmax of the previous
// tile follows the section "FlashAttention-3" (matmul/softmax interleaving),
// realised here inside each wave's instruction stream.
//
// gfx950 design.  Three kernels share tiles, layouts and the epilogue:
//  * fwd_unit2_kernel (fa_fwd, d = 128, large grids): 8 waves x 64 query rows, each wave
//    two 32-row halves that share every K and V operand read (half the LDS reads per
//    product of the 32-row waves, and 512 rows served by each K/V tile loaded), two
//    waves per SIMD; per half the same steps, and bits, as fwd_unit_kernel.
//  * fwd_unit_kernel (fa_fwd otherwise, and the mask family without block lists): NW
//    waves x 32 query rows, each wave taking one 32-key unit at a time while the other
//    waves on its SIMD overlap its softmax with their products: at d = 128 12 waves (one
//    workgroup per CU, three waves per SIMD), or 6 (two workgroups per CU) when the
//    384-row grid would leave CUs idle; at d = 64 8 waves, two workgroups per CU (four
//    waves per SIMD).  On the smallest grids (no key split asked for) it runs two waves
//    per 32 queries, each taking one 32-key unit of every tile, merged at the end: 8
//    waves on 128 rows at d = 128, 4 on 64 or 6 on 96 rows at d = 64.
//  * fwd_kernel (the mask family, fa_fwd_masked): 8 waves x 32 rows (256-row blocks,
//    the granularity of the block lists), two waves per SIMD, with a software
//    pipeline per wave: the products S_{u+1} = K_{u+1} Q^T are issued while the
//    softmax of unit u runs, then O^T += V_u^T P_u; the two waves of a SIMD run half a
//    unit apart.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: every
//    lane holds the scores of ONE query (lane % 32) for 32 keys, so the row max
//    and row sum are in-lane plus one permlane32 swap, and the probabilities are
//    already in the B-operand layout of O^T += V^T P^T (no LDS round trip).  The
//    key order inside each 16-key MFMA step is permuted consistently on both
//    operands, which the sum over keys does not see.
//  * Q stays in VGPRs for the whole key loop.  K and V tiles of 64 keys go from
//    HBM straight into LDS (buffer loads to LDS, 16 bytes per lane, into slots that
//    are distinct LDS objects indexed at compile time: three slots and two tiles in
//    flight, or two slots and one where two workgroups share a CU).
//    Rows are padded to a pitch of row+16 bytes for K and
//    row+64 bytes for V: with the 64 four-byte banks of the CDNA4 LDS, 16 lanes
//    reading 16 bytes from 16 consecutive K rows, and 32 lanes reading 8 bytes
//    from 4 consecutive V rows (ds_read_b64_tr_b16), then hit distinct banks
//    (measured free of bank conflicts), and every LDS address is a lane
//    constant plus an immediate.  The loads use buffer descriptors that end at
//    row N, so rows past the sequence end land as zeros.
//  * Scores are kept in log2 units.  fwd_kernel raises the reference max only when a
//    row's max exceeds it by more than 8 (so P <= 256), and rescales O only when
//    some lane of the wave raised it.  fwd_unit_kernel forms no row max at all on its
//    common path: P comes from the reference as it stands, and only when a lane's
//    probabilities over the unit sum past 256 (or the lane has no reference yet)
//    does the wave take the row max, raise the reference (in bf16 to 8 above that max,
//    so that rising scores come back to this path half as often) and form P again; its
//    products run at raised wave priority (s_setprio), so a wave entering them is
//    issued ahead of waves still in their softmax.
//  * Causal: a workgroup stops at the last tile its rows can see; units no query of a
//    wave sees are skipped by that wave (fwd_unit_kernel) or add only zeros in a
//    masked variant without branches (fwd_kernel).
//  * Block ids are remapped so that all query blocks sharing a K/V head run on
//    one XCD (block ids are dealt round-robin over the 8 XCDs) and the longest
//    causal blocks start first.
#include <cfloat>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// GEN = the mask family: per-sequence lengths (packed or fixed, queries and keys of
// different lengths, bottom-right aligned), a window (left, right) and optional
// block lists of key tiles; CAUSAL is then unused (causal is the window (-1, 0)).
template <class Tag, int D, bool CAUSAL, bool GEN = false>
__global__ void __launch_bounds__(512) fwd_kernel(const FwdArgs a) {
  using E = Elt<Tag>;
  constexpr int NW = 8;                 // waves per workgroup
  constexpr int BR = 32 * NW;           // query rows per workgroup
  constexpr int BC = 64;                // keys per tile
  constexpr int ROWB = D * 2;           // bytes of one row
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int PK = ROWB + 16;         // LDS pitch of K rows (16-byte row reads)
  constexpr int PV = ROWB + 64;         // LDS pitch of V rows (transposing reads)
  using Tiles = TilePair<ROWB, PK, PV, NW>;
  constexpr int KBYTES = Tiles::ABYTES;
  constexpr int SLOT = Tiles::SLOT;
  constexpr int IPW = Tiles::IPW;
  constexpr int NE = D / 32;            // 32-row blocks of O^T
  constexpr int NS = D / 16;            // k-steps of S^T
  constexpr float TAU = 8.f;            // rescale threshold (log2 units)
  constexpr int PD = 2;                 // LDS read-ahead, in MFMA slots (3 and 4 measured no faster)
  static_assert(PD <= NS && PD <= 2 * NE, "read-ahead within one phase");

  // Three slots as distinct LDS objects: tile j uses slot j % 3, known at compile time
  // in the 3-tile unrolled loops, so the compiler can tell that the loads into one slot
  // leave the others alone and does not make their reads wait for those loads.
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

  int b, hq, iq;
  map_q_block(((GEN ? a.maxq : N) + BR - 1) / BR, a.B, a.Hq, a.Hkv, b, hq, iq);
  const int hkv = hq / (a.Hq / a.Hkv);
  // sequence geometry: Lq queries, Lk keys; first row of this head's sequence
  int Lq = N, Lk = N;
  size_t qhead, kvhead;
  if constexpr (GEN) {
    if (a.cu_q != nullptr) {   // packed; offsets clamped to the tensors whatever the lengths say
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
  const unsigned char* Qg = (const unsigned char*)a.q + qhead * ROWB;
  const unsigned char* Kg = (const unsigned char*)a.k + kvhead * ROWB;
  const unsigned char* Vg = (const unsigned char*)a.v + kvhead * ROWB;

  const int q0 = iq * BR;
  if (GEN && q0 >= Lq) return;   // the whole workgroup: past this sequence's queries
  const int qw = q0 + wave * 32;   // first row of this wave
  const int myq = qw + r32;        // the query this lane's scores belong to

  // Q^T as the B operand: lane holds Q[myq][16s + 8hh .. +7]
  u32x4 qf[NS];
  if (myq < Lq) {
    const unsigned char* qp = Qg + (size_t)myq * ROWB + 16 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const u32x4*)(qp + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = u32x4{0, 0, 0, 0};
  }

  const int nkv = (Lk + BC - 1) / BC;
  // Key tiles visited, in order: tile_of(j), j < ntile.  The mask family visits the tiles
  // of the workgroup's key interval [klo, khi] (union over its queries of each query's
  // window), filtered by the block list when there is one.
  const int off = Lk - Lq;                  // query i sits at key position i + off
  const int qlast = min(q0 + BR, Lq) - 1;
  int ntile, t_lo = 0, p0 = 0;
  const int* lst = nullptr;
  int lo_q = 0, hi_q = Lk - 1;              // this lane's visible key interval
  int JH = 0, JT = 0;                       // masked head [0, JH), plain [JH, JT), masked tail
  if constexpr (GEN) {
    auto lo_of = [&](int i) { return a.wl >= 0 ? i + off - a.wl : 0; };
    auto hi_of = [&](int i) { return a.wr >= 0 ? min(i + off + a.wr, Lk - 1) : Lk - 1; };
    lo_q = lo_of(myq);
    hi_q = hi_of(myq);
    const int klo = max(lo_of(q0), 0), khi = hi_of(qlast);
    t_lo = klo / BC;
    const int t_hi = (Lk <= 0 || khi < klo) ? t_lo : khi / BC + 1;
    // tiles that need element masks: below the largest lower bound, or past the smallest
    // upper bound (which includes the tile holding key Lk-1 when Lk is ragged)
    const int tm_head = (max(lo_of(qlast), 0) + BC - 1) / BC;     // tiles < tm_head
    const int tm_tail = (hi_of(q0) + 1) / BC;                       // tiles >= tm_tail
    int P1, P2;
    if (a.bidx != nullptr) {
      const int hm = a.bheads == 1 ? 0 : hq;
      const size_t row = ((size_t)b * a.bheads + hm) * a.bnq + iq;
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
    // tile j's mask flag covers its second unit and the next tile's first unit
    JH = min(ntile, (P1 + 2) / 3 * 3);
    JT = max(JH, max(P2 - 1, 0) / 3 * 3);
  } else {
    ntile = CAUSAL ? min(nkv, (min(q0 + BR, N) - 1) / BC + 1) : nkv;
  }
  // tile index of list position j; past the list, the first tile past the keys (masked)
  auto tile_of = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (!GEN) return j;
    if (j >= ntile) return nkv;
    if (lst == nullptr) return t_lo + j;
    return min(max(lst[p0 + j], t_lo), nkv - 1);
  };

  // ---- HBM -> LDS: tile t of K and V into slot sl ----
  int doff[IPW];
  Tiles::offsets(wave, lane, doff);
  auto dma = [&](int t, unsigned char* sl) __attribute__((always_inline)) {
    Tiles::load(Kg, Vg, Lk, t, wave, doff, sl);
  };

  // ---- per-lane LDS offsets (plus immediates) ----
  // K (A operand of S^T): row 32c + r32, chunk 2st + hh
  const int ka = r32 * PK + 16 * hh;
  // V (A operand of O^T, read transposed): row 16t + 8u + R, element 32e + 16x + 4y
  const int va = KBYTES + (4 * hh + ((lane & 15) >> 2)) * PV + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  const float c2 = a.scale_log2;
  float mr = -INFINITY;       // reference max of query myq (log2 units)
  float l_run = 0.f;          // running sum over this lane's half of the keys
  f32x16 o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[e][v] = 0.f;

  // The pipeline works on 32-key units: unit 2j + h is half h of tile j.
  auto kread = [&](const unsigned char* sl, int h, int st) __attribute__((always_inline)) {
    return *(const u32x4*)(sl + h * 32 * PK + ka + 32 * st);
  };
  auto vread = [&](const unsigned char* sl, int hv, int h, int e) __attribute__((always_inline)) {
    const unsigned char* p = sl + hv * 32 * PV + va;
    return cat(lds_read_tr(p + 16 * h * PV + 64 * e), lds_read_tr(p + (16 * h + 8) * PV + 64 * e));
  };

  auto rowmax16 = [&](const f32x16& s) __attribute__((always_inline)) {
    float mx = s[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
    return mx;
  };
  // new reference from the unit's row max; returns alpha = exp2(old - new), sets mref
  auto newref = [&](float mx, bool& raise, float& mref) __attribute__((always_inline)) {
    mx *= c2;
    raise = mx > mr + TAU;
    const float mnew = raise ? mx : mr;
    const float alpha = (mr == -INFINITY) ? 0.f : fast_exp2(mr - mnew);
    mref = (mnew == -INFINITY) ? 0.f : mnew;
    mr = mnew;
    return alpha;
  };
  auto packp = [&](const f32x16& s, int h) __attribute__((always_inline)) {
    return u32x4{E::pack(s[8 * h + 0], s[8 * h + 1]), E::pack(s[8 * h + 2], s[8 * h + 3]),
                 E::pack(s[8 * h + 4], s[8 * h + 5]), E::pack(s[8 * h + 6], s[8 * h + 7])};
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[e][v] *= alpha;
  };

  // K fragments of the next unit's first two k-steps, read ahead
  u32x4 kpre[PD];

  // Unit u, hand-scheduled in two phases.
  // S-phase (scores of unit u in sc, its reference max already chosen): NS slots, each
  // one MFMA of S_{u+1} (K in half hn of slot sln) plus two of unit u's exponentials;
  // ends with P packed and O rescaled if unit u raised the reference.
  // PV-phase (V in half hc of slot slc): 2*NE slots, each one MFMA of O^T += V^T P plus
  // two adds of the row sum, and the row max of S_{u+1} (masked first under MASK: keys
  // past N or, causal, after the query), which picks unit u+1's reference; its last PD
  // slots read unit u+2's first K fragments (half hp of slot slp).
  // LDS reads run PD slots ahead.
  struct Ref {
    float mref;    // reference max (log2 units) the exponentials subtract
    float alpha;   // exp2(previous reference - mref)
    bool raise;    // this lane raised the reference
  };
  struct Pend {
    u32x4 pf[2];   // P of the unit, packed B operands of the two 16-key steps
    u32x4 vpre[PD];  // first PD V fragments of the PV-phase
  };
  // Keys every query of this wave sees: [wlo, whi] (wave-uniform); a unit inside it needs
  // no per-element mask.
  int wlo = 0, whi;
  if constexpr (GEN) {
    wlo = a.wl >= 0 ? max(min(qw + 31, Lq - 1) + off - a.wl, 0) : 0;
    whi = a.wr >= 0 ? min(qw + off + a.wr, Lk - 1) : Lk - 1;
  } else {
    whi = CAUSAL ? min(qw, N - 1) : N - 1;
  }
  // unit u's first key: half u % 2 of tile tile_of(u / 2)
  auto mask_unit = [&](int u, f32x16& s) __attribute__((always_inline)) {
    const int k0 = GEN ? tile_of(u >> 1) * BC + 32 * (u & 1) : u * 32;
    if (k0 >= wlo && k0 + 31 <= whi) return;
    int lim = (GEN ? min(Lk, hi_q + 1) : N) - k0 - 4 * hh;   // key offset limit (exclusive)
    if (!GEN && CAUSAL) lim = min(lim, myq - k0 - 4 * hh + 1);
    const int llo = lo_q - k0 - 4 * hh;                       // first visible offset (GEN)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int o = 8 * (v >> 2) + (v & 3);
      if (o >= lim || (GEN && o < llo)) s[v] = -INFINITY;
    }
  };
  auto sphase = [&](const unsigned char* slc, int hc, const unsigned char* sln, int hn, f32x16& sc,
                    f32x16& sn, const Ref& rf, Pend& pd) __attribute__((always_inline)) {
    u32x4 kf[NS];
#pragma unroll
    for (int i = 0; i < PD; ++i) kf[i] = kpre[i];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k == 0) sn = zero16();
      sn = E::mma(kf[k], qf[k], sn);
      if (k + PD < NS) kf[k + PD] = kread(sln, hn, k + PD);
      else pd.vpre[k + PD - NS] = vread(slc, hc, (k + PD - NS) / NE, (k + PD - NS) % NE);
#pragma unroll
      for (int v = (16 * k) / NS; v < (16 * (k + 1)) / NS; ++v) {
        sc[v] = fast_exp2(fmaf(sc[v], c2, -rf.mref));
        keep(sc[v]);   // stays in this slot (no sinking past the rescale branch)
      }
      if (k == NS - 1) {
        pd.pf[0] = packp(sc, 0);
        pd.pf[1] = packp(sc, 1);
        keep(pd.pf[0]);
        keep(pd.pf[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_amdgcn_ballot_w64(rf.raise) != 0) rescale(rf.alpha);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto pphase = [&](auto MASK, int u, const unsigned char* slc, int hc, const unsigned char* slp, int hp,
                    const f32x16& sc, f32x16& sn, Ref& rf, const Pend& pd) __attribute__((always_inline)) {
    u32x4 vf[2 * NE];
#pragma unroll
    for (int i = 0; i < PD; ++i) vf[i] = pd.vpre[i];
    float rs = 0.f, mx = 0.f;
    const float alpha = rf.alpha;
#pragma unroll
    for (int k = 0; k < 2 * NE; ++k) {
      const int h = k / NE, e = k % NE;
      o[e] = E::mma(vf[k], pd.pf[h], o[e]);
      if (k + PD < 2 * NE) vf[k + PD] = vread(slc, hc, (k + PD) / NE, (k + PD) % NE);
      else kpre[k + PD - 2 * NE] = kread(slp, hp, k + PD - 2 * NE);
      // row sum of the fp32 P (the saved LSE needs it to fp32 accuracy), in this slot
#pragma unroll
      for (int v = (16 * k) / (2 * NE); v < (16 * (k + 1)) / (2 * NE); ++v) rs += sc[v];
      keep(rs);
      // row max of the next unit's scores (their last MFMA was the S-phase's last slot)
      if (k == 1) {
        if constexpr (decltype(MASK)::value) mask_unit(u + 1, sn);
        mx = fmaxf(fmaxf(sn[0], sn[1]), fmaxf(sn[2], sn[3]));
#pragma unroll
        for (int v = 4; v < 8; ++v) mx = fmaxf(mx, sn[v]);
        keep(mx);
      }
      if (k == 2) {
#pragma unroll
        for (int v = 8; v < 16; ++v) mx = fmaxf(mx, sn[v]);
        mx = half_max(mx);
        keep(mx);
      }
      if (k == 3) {
        rf.alpha = newref(mx, rf.raise, rf.mref);
        keep(rf.alpha);
        keep(rf.mref);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = fmaf(l_run, alpha, rs);
    keep(l_run);
  };

  // ---- pipeline: two tiles in flight in LDS; S of unit u+1 formed during softmax of u ----
  // The two waves that share a SIMD (w and w + 4) run half a unit apart: the second
  // group (LATE) passes each tile barrier after, not before, the S-phase of the tile's
  // first unit, so one wave's softmax runs while the other's PV products keep the
  // matrix core busy (the FA3 section's ping-pong between warpgroups, on one SIMD).
  // With three slots this is safe: nothing reads tile j-1 after barrier j, and the
  // early S-phase reads only tile j, published at barrier j-1.
  f32x16 sa, sb;
  Ref rf;
  // Tile j (slot T = j % 3): sync, load tile j+2, units 2j (scores in sa) and 2j+1 (sb).
  // MASK masks the units after this tile's first (the first was masked, if needed, by
  // the phase before it).  The products of the unit after the last are formed from a
  // valid slot and never used (masked: the last tile always runs masked).
  auto tile = [&](auto Tc, auto MASK, auto LATE, int j) __attribute__((always_inline)) {
    constexpr int T = decltype(Tc)::value;
    unsigned char* const sc = slot(T);
    unsigned char* const sn = slot((T + 1) % 3);
    Pend p0, p1;
    if constexpr (decltype(LATE)::value) sphase(sc, 0, sc, 1, sa, sb, rf, p0);
    if (j > 0) {
      wait_loads();      // this wave's loads of tile j+1 landed
      __syncthreads();   // everyone's; slot (j-1)%3 is free
    }
    if (j + 2 < ntile) dma(tile_of(j + 2), slot((T + 2) % 3));
    if constexpr (!decltype(LATE)::value) sphase(sc, 0, sc, 1, sa, sb, rf, p0);
    pphase(MASK, 2 * j, sc, 0, sn, 0, sa, sb, rf, p0);
    sphase(sc, 1, sn, 0, sb, sa, rf, p1);
    pphase(MASK, 2 * j + 1, sc, 1, sn, 1, sb, sa, rf, p1);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using Plain = std::false_type;
  using Masked = std::true_type;

  if (!GEN || ntile > 0) {   // (a mask-family workgroup may have no tile to visit)
  dma(tile_of(0), slot0);
  if (ntile > 1) dma(tile_of(1), slot1);
  wait_loads();
  __syncthreads();
  sa = zero16();
#pragma unroll
  for (int st = 0; st < NS; ++st) sa = E::mma(kread(slot0, 0, st), qf[st], sa);
#pragma unroll
  for (int i = 0; i < PD; ++i) kpre[i] = kread(slot0, 1, i);
  mask_unit(0, sa);
  rf.alpha = newref(half_max(rowmax16(sa)), rf.raise, rf.mref);
  // Tiles whose units, and the unit after them, all precede every wave's last unit (the
  // one holding its diagonal when causal, or the last key) need no mask.
  if constexpr (!GEN) {
    const int ulast0 = (CAUSAL ? min(q0 + 31, N - 1) : N - 1) / 32;
    JT = min(ntile, max(ulast0 - 1, 0) / 2) / 3 * 3;
  }
  auto run = [&](auto LATE) __attribute__((always_inline)) {
    int j = 0;
    if constexpr (GEN) {
      for (; j < JH; j += 3) {
        tile(I0{}, Masked{}, LATE, j);
        if (j + 1 >= ntile) break;
        tile(I1{}, Masked{}, LATE, j + 1);
        if (j + 2 >= ntile) break;
        tile(I2{}, Masked{}, LATE, j + 2);
      }
      j = JH;
    }
    for (; j < JT; j += 3) {
      tile(I0{}, Plain{}, LATE, j);
      tile(I1{}, Plain{}, LATE, j + 1);
      tile(I2{}, Plain{}, LATE, j + 2);
    }
    for (; j < ntile; j += 3) {
      tile(I0{}, Masked{}, LATE, j);
      if (j + 1 >= ntile) break;
      tile(I1{}, Masked{}, LATE, j + 1);
      if (j + 2 >= ntile) break;
      tile(I2{}, Masked{}, LATE, j + 2);
    }
  };
  if (wave >= NW / 2) run(std::true_type{});
  else run(std::false_type{});
  }

  // epilogue: O = O^T / l, LSE = ln(2) * (m + log2 l); a row that saw no key (mask
  // family only) gets O = 0 and LSE = -inf
  const float l_tot = half_sum(l_run);
  if (myq < Lq) {
    const float inv = (GEN && !(l_tot > 0.f)) ? 0.f : 1.f / l_tot;
    store_row16<E>((unsigned char*)a.o + (qhead + myq) * ROWB, o, inv, hh);
    if (hh == 0) a.lse[qhead + myq] = (GEN && !(l_tot > 0.f)) ? -INFINITY : (mr + log2f(l_tot)) * kLn2;
  }
}

// The forward without block lists: NW waves of 32 queries, each taking one 32-key
// unit at a time — scores, mask, exponentials and row sum (the reference max only on
// the rare slow path), then O^T += V^T P^T at raised wave priority — with no software
// pipeline: the other waves on the SIMD overlap one wave's softmax with their
// products.  Without the pipeline's second unit a wave needs ~156 registers at d = 128
// (three waves per SIMD) and ~105 at d = 64 (four).  Below 12 waves (6 at d = 128, 8
// at d = 64) two LDS slots (75 KB at d = 128, 43 KB at d = 64) leave room for a
// second workgroup per CU; at 12 three slots keep two tiles in flight.  Same tiles,
// loads, layouts and epilogue as fwd_kernel; the reference max is kept differently
// (above), so the two kernels agree to rounding, not bit for bit.  With KS = 1 the
// arithmetic is the same at every NW, and a unit that no query of a wave sees (past its diagonal,
// outside its window) is skipped by that wave, which changes no bit.  GEN: the mask
// family without block lists (lengths, packed batches, windows) as in fwd_kernel.
// KS = 2 (small grids): two waves per 32 queries, one taking the first and one the second
// 32-key unit of every tile, their O, row sums and references merged through LDS at the
// end (the online softmax's merge of two partial results, "FlashAttention Primer",
// "FlashAttention-1"; the key split of Flash-Decoding, "Flash Attention" wiki), so a
// block's chain of units is half as long and its rows spread over more, smaller workgroups.
// The d = 64 4-wave form of it (two workgroups per CU, one wave per SIMD each) reads every
// K and V operand of a unit before its products, with the registers of two waves per SIMD
// (12-17 % faster there; no gain at d = 128, and the 6-wave form would spill).
constexpr int unit_waves_per_eu(int d, int nw, int ks) { return (ks == 2 && d == 64 && nw == 4) ? 2 : d == 128 ? 3 : 4; }
template <class Tag, int D, bool CAUSAL, int NW, bool GEN = false, int KS = 1>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(unit_waves_per_eu(D, NW, KS))))
fwd_unit_kernel(const FwdArgs a) {
  using E = Elt<Tag>;
  static_assert(KS == 1 || KS == 2, "one or two waves per 32 queries");
  constexpr int RG = NW / KS;   // 32-query row groups of the workgroup
  constexpr bool PREREAD = KS == 2 && D == 64 && NW == 4;   // all operands of a unit up front
  constexpr int BR = 32 * RG;
  constexpr int BC = 64;
  constexpr int ROWB = D * 2;
  // K and V tiles free of bank conflicts for the row reads of K and the transposing reads
  // of V: at d = 64 unpadded with their 16-byte chunks XOR-swizzled (fa_tiles.h), 20 %
  // fewer tile loads (up to 2.4 % faster); at d = 128 padded (K row+16 B, V row+64 B), since
  // the swizzled addresses take ~12 more registers a wave there and cost 1.5-2.7 %
  constexpr bool SWZ = D == 64;
  constexpr int PK = SWZ ? ROWB : ROWB + 16;
  constexpr int PV = SWZ ? ROWB : ROWB + 64;
  using Tiles = TilePair<ROWB, PK, PV, NW, SWZ, SWZ>;
  using SO = SwzOffsets<ROWB>;
  constexpr int KBYTES = Tiles::ABYTES;
  constexpr int SLOT = Tiles::SLOT;
  constexpr int IPW = Tiles::IPW;
  constexpr int NE = D / 32;
  constexpr int NS = D / 16;
  constexpr float TAU_SUM = 256.f;   // bound on a lane's sum of P over a unit (2^8)
  // a raised reference sits HEADROOM (log2 units) above the row max that raised it: scores
  // that keep rising then have to climb about 16 log2 units, not 8, before P's sum passes
  // TAU_SUM again.  bf16 only: P scaled down that far would reach fp16's subnormal range
  constexpr float HEADROOM = std::is_same<Tag, bf16_tag>::value ? 8.f : 0.f;
  // NSL LDS slots as distinct objects (see fwd_kernel): three with one workgroup per
  // CU (12 waves, or the key-split workgroups of small grids), two where a second
  // workgroup has to fit beside it
  constexpr int NSL = (NW >= 12 || KS == 2) ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[NSL == 3 ? SLOT : 1];
  auto slot = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? slot0 : i == 1 ? slot1 : slot2;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rgw = KS == 1 ? wave : wave % RG;   // this wave's row group
  const int kh = KS == 1 ? 0 : wave / RG;       // KS = 2: the unit of each tile it takes
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;
  int b, hq, iq;
  // key split: consecutive blocks are the splits of one query block
  const int ks = GEN ? a.ksplit : 1;
  const int sidx = ks > 1 ? (int)blockIdx.x % ks : 0;
  map_q_block(((GEN ? a.maxq : N) + BR - 1) / BR, a.B, a.Hq, a.Hkv, b, hq, iq, (int)blockIdx.x / ks);
  const int hkv = hq / (a.Hq / a.Hkv);
  // sequence geometry: Lq queries, Lk keys (offsets clamped to the tensors)
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
  const unsigned char* Qg = (const unsigned char*)a.q + qhead * ROWB;
  const unsigned char* Kg = (const unsigned char*)a.k + kvhead * ROWB;
  const unsigned char* Vg = (const unsigned char*)a.v + kvhead * ROWB;
  const int q0 = iq * BR;
  if (GEN && q0 >= Lq) return;   // the whole workgroup: past this sequence's queries
  const int qw = q0 + rgw * 32;
  const int myq = qw + r32;
  u32x4 qf[NS];
  if (myq < Lq) {
    const unsigned char* qp = Qg + (size_t)myq * ROWB + 16 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = *(const u32x4*)(qp + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = u32x4{0, 0, 0, 0};
  }
  // Key tiles t_lo .. t_lo + ntile - 1 (the union of the workgroup's queries' windows);
  // keys some query of this wave sees: [ulo, uhi] (empty when the wave has no query);
  // keys every query of it sees: [wlo, whi]; this lane's: [lo_q, hi_q].
  const int off = Lk - Lq;   // query i sits at key position i + off
  int t_lo = 0, ntile, ulo = 0, uhi, wlo = 0, whi, lo_q = 0, hi_q = Lk - 1;
  if constexpr (GEN) {
    auto lo_of = [&](int i) { return a.wl >= 0 ? i + off - a.wl : 0; };
    auto hi_of = [&](int i) { return a.wr >= 0 ? min(i + off + a.wr, Lk - 1) : Lk - 1; };
    const int qlw = min(qw + 31, Lq - 1), qlast = min(q0 + BR, Lq) - 1;
    lo_q = lo_of(myq);
    hi_q = hi_of(myq);
    ulo = max(lo_of(qw), 0);
    uhi = qw >= Lq ? -1 : hi_of(qlw);
    wlo = max(lo_of(qlw), 0);
    whi = hi_of(qw);
    int klo = max(lo_of(q0), 0), khi = hi_of(qlast);
    if (ks > 1) {   // this split's keys only (64-key aligned, so whole units)
      const int kb = sidx * a.kchunk, ke = min(kb + a.kchunk, Lk) - 1;
      lo_q = max(lo_q, kb);
      hi_q = min(hi_q, ke);
      ulo = max(ulo, kb);
      uhi = min(uhi, ke);
      wlo = max(wlo, kb);
      whi = min(whi, ke);
      klo = max(klo, kb);
      khi = min(khi, ke);
    }
    t_lo = klo / BC;
    ntile = (Lk <= 0 || khi < klo) ? 0 : khi / BC + 1 - t_lo;
  } else {
    const int nkv = (N + BC - 1) / BC;
    ntile = CAUSAL ? min(nkv, (min(q0 + BR, N) - 1) / BC + 1) : nkv;
    uhi = qw >= N ? -1 : CAUSAL ? min(qw + 31, N - 1) : N - 1;
    whi = CAUSAL ? min(qw, N - 1) : N - 1;
  }
  // K rows 32h + r32, chunk 2st + hh (A operand of S^T); V read transposed, rows
  // 32hv + 16h + 8u + R (A operand of O^T): the operands of fwd_kernel, from swizzled rows
  int doff[IPW];
  Tiles::offsets(wave, lane, doff);
  const int ka = SWZ ? SO::rows_a0(lane) : r32 * PK + 16 * hh;
  const int va = KBYTES + (SWZ ? SO::tr_lane(lane)
                               : (4 * hh + ((lane & 15) >> 2)) * PV + 32 * ((lane >> 4) & 1) + 8 * (lane & 3));
  auto kread = [&](const unsigned char* sl, int h, int st) __attribute__((always_inline)) {
    if constexpr (SWZ) return *(const u32x4*)(sl + h * 32 * PK + (ka ^ (st << 5)));
    else return *(const u32x4*)(sl + h * 32 * PK + ka + 32 * st);
  };
  auto vread = [&](const unsigned char* sl, int hv, int h, int e) __attribute__((always_inline)) {
    const unsigned char* p = sl + (32 * hv + 16 * h) * PV;
    if constexpr (SWZ)
      return cat(lds_read_tr(p + (va ^ SO::tr_inst(e, 0))), lds_read_tr(p + 8 * PV + (va ^ SO::tr_inst(e, 1))));
    else
      return cat(lds_read_tr(p + va + 64 * e), lds_read_tr(p + 8 * PV + va + 64 * e));
  };
  const float c2 = a.scale_log2;
  float mr = -FLT_MAX, l_run = 0.f;   // reference (log2 units); -FLT_MAX: none yet
  f32x16 o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[e][v] = 0.f;
  // unit u = keys 32u .. 32u+31, half h of the tile in slot sl
  auto unit = [&](int u, const unsigned char* sl, int h) __attribute__((always_inline)) {
    const int k0 = u * 32;
    if (k0 > uhi || k0 + 31 < ulo) return;   // wave-uniform: no query of this wave sees these keys
    f32x16 s;
    u32x4 vall[PREREAD ? 2 * NE : 1];
    u32x4 vf;
    if constexpr (PREREAD) {
      u32x4 kall[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st) kall[st] = kread(sl, h, st);
#pragma unroll
      for (int st = 0; st < NS; ++st) s = E::mma(kall[st], qf[st], st == 0 ? zero16() : s);
#pragma unroll
      for (int k = 0; k < 2 * NE; ++k) vall[k] = vread(sl, h, k / NE, k % NE);
    } else {
      u32x4 kf = kread(sl, h, 0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const u32x4 kc = kf;
        if (st + 1 < NS) kf = kread(sl, h, st + 1);
        s = E::mma(kc, qf[st], st == 0 ? zero16() : s);
      }
      vf = vread(sl, h, 0, 0);   // first PV operand, read while the scores settle
    }
    if (!(k0 >= wlo && k0 + 31 <= whi)) {   // keys outside this lane's window or past the end: -inf
      int lim = (GEN ? min(Lk, hi_q + 1) : N) - k0 - 4 * hh;
      if (!GEN && CAUSAL) lim = min(lim, myq - k0 - 4 * hh + 1);
      const int llo = lo_q - k0 - 4 * hh;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int oo = 8 * (v >> 2) + (v & 3);
        if (oo >= lim || (GEN && oo < llo)) s[v] = -INFINITY;
      }
    }
    // P from the reference as it stands, with no row max: any reference gives the same
    // normalised result, it only has to keep P from overflowing.  If this lane's
    // probabilities sum past TAU_SUM = 2^8 (so some P may exceed 2^8, or the lane has no
    // reference yet, whose sentinel -FLT_MAX makes every visible P infinite), the wave
    // takes the slow path: the row max of the unit, the reference raised to it (plus
    // HEADROOM), O and the row sum rescaled, P formed again.  Masked scores (-inf) give
    // P = 0 either way.
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(s[v], c2, -mr));
    auto rowsum = [&]() __attribute__((always_inline)) {
      float t[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) t[v] = p[2 * v] + p[2 * v + 1];
#pragma unroll
      for (int v = 0; v < 4; ++v) t[v] = t[2 * v] + t[2 * v + 1];
      return (t[0] + t[1]) + (t[2] + t[3]);
    };
    float rs = rowsum();
    if (__builtin_amdgcn_ballot_w64(!(rs <= TAU_SUM)) != 0) {
      float mx = s[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
      const float mnew = fmaxf(mr, half_max(mx) * c2 + HEADROOM);
      const float alpha = fast_exp2(mr - mnew);   // 0 from the sentinel, 1 if unmoved
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[e][v] *= alpha;
      l_run *= alpha;
      mr = mnew;
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(s[v], c2, -mr));
      rs = rowsum();
    }
    l_run += rs;
    const u32x4 pf[2] = {
        u32x4{E::pack(p[0], p[1]), E::pack(p[2], p[3]), E::pack(p[4], p[5]), E::pack(p[6], p[7])},
        u32x4{E::pack(p[8], p[9]), E::pack(p[10], p[11]), E::pack(p[12], p[13]), E::pack(p[14], p[15])}};
    // the products go first on the SIMD: a wave entering them takes the issue slots from
    // waves still in their softmax, which keeps the matrix core fed
    __builtin_amdgcn_s_setprio(1);
    if constexpr (PREREAD) {
#pragma unroll
      for (int k = 0; k < 2 * NE; ++k) o[k % NE] = E::mma(vall[k], pf[k / NE], o[k % NE]);
    } else {
#pragma unroll
      for (int k = 0; k < 2 * NE; ++k) {
        const int t = k / NE, e = k % NE;
        const u32x4 vc = vf;
        if (k + 1 < 2 * NE) vf = vread(sl, h, (k + 1) / NE, (k + 1) % NE);
        o[e] = E::mma(vc, pf[t], o[e]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto dma = [&](int j, unsigned char* sl) __attribute__((always_inline)) {
    Tiles::load(Kg, Vg, Lk, t_lo + j, wave, doff, sl);
  };
  // tile j in slot j % NSL: sync, load tile j + NSL - 1 into the slot tile j-1 used,
  // its two units
  auto tile = [&](auto Tc, int j) __attribute__((always_inline)) {
    constexpr int T = decltype(Tc)::value;
    unsigned char* const sc = slot(T);
    if (j > 0) {
      wait_loads();      // this wave's loads of tile j landed
      __syncthreads();   // everyone's; everyone is done with tile j-1
    }
    if (j + NSL - 1 < ntile) dma(j + NSL - 1, slot((T + NSL - 1) % NSL));
    if constexpr (KS == 1) {
      unit(2 * (t_lo + j), sc, 0);
      unit(2 * (t_lo + j) + 1, sc, 1);
    } else {
      unit(2 * (t_lo + j) + kh, sc, kh);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if (!GEN || ntile > 0) {   // (a mask-family workgroup may have no tile to visit)
    dma(0, slot0);
    if (NSL == 3 && ntile > 1) dma(1, slot1);
    wait_loads();
    __syncthreads();
    for (int j = 0; j < ntile; j += NSL) {
      tile(I0{}, j);
      if (j + 1 >= ntile) break;
      tile(I1{}, j + 1);
      if constexpr (NSL == 3) {
        if (j + 2 >= ntile) break;
        tile(I2{}, j + 2);
      }
    }
  }
  if constexpr (KS == 2) {
    // the second-unit wave hands its O^T, reference and row sum (lane for lane: both
    // waves hold the same rows in the same layout) to the first, which rescales both to
    // the larger reference and adds them; as many row groups' records per LDS slot as fit
    constexpr int REC = (NE * 16 + 2) * 64;   // floats
    constexpr int RPS = SLOT / (REC * 4);     // records per slot
    static_assert(RPS >= 1 && RG <= RPS * NSL, "the merge records fit the slots");
    __syncthreads();   // every wave is done with the last tile
    float* const rec = (float*)slot((unsigned)rgw / RPS) + ((unsigned)rgw % RPS) * REC + lane;
    if (kh == 1) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int v = 0; v < 16; ++v) rec[(16 * e + v) * 64] = o[e][v];
      rec[NE * 16 * 64] = mr;
      rec[(NE * 16 + 1) * 64] = l_run;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = rec[NE * 16 * 64], l1 = rec[(NE * 16 + 1) * 64];
    const float mm = fmaxf(mr, m1);
    const float a0 = fast_exp2(mr - mm), a1 = fast_exp2(m1 - mm);   // 0 for a part with no key
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[e][v] = o[e][v] * a0 + rec[(16 * e + v) * 64] * a1;
    l_run = l_run * a0 + l1 * a1;
    mr = mm;
  }
  // epilogue: O = O^T / l, LSE = ln(2) * (m + log2 l); a row that saw no key (mask
  // family only) gets O = 0 and LSE = -inf
  const float l_tot = half_sum(l_run);
  if (GEN && ks > 1) {   // this split's part of the row: O / l in fp32 and its LSE
    if (myq < Lq) {
      const float inv = !(l_tot > 0.f) ? 0.f : 1.f / l_tot;
      const size_t part = (qhead + myq) * (size_t)ks + sidx;
      float* op = a.opart + part * D;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * e + 8 * g + 4 * hh;
          *(f32x4*)(op + d0) = f32x4{o[e][4 * g] * inv, o[e][4 * g + 1] * inv, o[e][4 * g + 2] * inv,
                                     o[e][4 * g + 3] * inv};
        }
      if (hh == 0) a.lpart[part] = !(l_tot > 0.f) ? -INFINITY : (mr + log2f(l_tot)) * kLn2;
    }
    return;
  }
  if (myq < Lq) {
    const float inv = (GEN && !(l_tot > 0.f)) ? 0.f : 1.f / l_tot;
    // 16 bytes a lane (store_row16: the two lanes of the row swap an 8-byte piece)
    store_row16<E>((unsigned char*)a.o + (qhead + myq) * ROWB, o, inv, hh);
    if (hh == 0) a.lse[qhead + myq] = (GEN && !(l_tot > 0.f)) ? -INFINITY : (mr + log2f(l_tot)) * kLn2;
  }
}


// The dense forward with 64 queries a wave: two 32-query halves share every K and V
// operand read (half the LDS read instructions of fwd_unit_kernel per product) and the
// workgroup of NW waves covers 64 NW rows, so each K/V tile loaded serves more rows.
// The registers of two halves (O^T and Q of 64 rows, 192 of the 256 a wave has at two
// waves per SIMD) leave no room to keep the scores past the exponentials, so the rare
// slow path forms them again from the tile still in LDS.  Per half the steps are those
// of fwd_unit_kernel (stale reference, slow path past TAU_SUM, the same products in the
// same order; a unit that only the second half sees adds exact zeros to the first), so
// the two kernels agree bit for bit.
template <class Tag, int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
fwd_unit2_kernel(const FwdArgs a) {
  using E = Elt<Tag>;
  constexpr int BR = 64 * NW;
  constexpr int BC = 64;
  constexpr int ROWB = D * 2;
  static_assert(D == 128, "at d = 64 the 32-query kernel's four waves per SIMD are faster");
  constexpr int PK = ROWB + 16;   // padded K and V rows, as in fwd_unit_kernel at d = 128
  constexpr int PV = ROWB + 64;
  using Tiles = TilePair<ROWB, PK, PV, NW>;
  constexpr int KBYTES = Tiles::ABYTES;
  constexpr int SLOT = Tiles::SLOT;
  constexpr int IPW = Tiles::IPW;
  constexpr int NE = D / 32;
  constexpr int NS = D / 16;
  constexpr float TAU_SUM = 256.f;   // bound on a lane's sum of P over a unit (2^8)
  // a raised reference sits HEADROOM (log2 units) above the row max that raised it: scores
  // that keep rising then have to climb about 16 log2 units, not 8, before P's sum passes
  // TAU_SUM again.  bf16 only: P scaled down that far would reach fp16's subnormal range
  constexpr float HEADROOM = std::is_same<Tag, bf16_tag>::value ? 8.f : 0.f;
  constexpr int NSL = 3;
  __shared__ __attribute__((aligned(1024))) unsigned char slot0[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot1[SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char slot2[SLOT];
  // Q operands of the second half for steps QP .. NS-1 parked in LDS (16 bytes a lane,
  // each lane reading back only what it wrote): 4 (NS - QP) registers fewer a wave, which
  // with the scheduling barriers below keeps the kernel within 256 registers unspilled
  constexpr int QP = NS - 2;
  __shared__ __attribute__((aligned(1024))) unsigned char qpark[NW * (NS - QP) * 1024];
  auto slot = [&](int i) __attribute__((always_inline)) -> unsigned char* {
    return i == 0 ? slot0 : i == 1 ? slot1 : slot2;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5, r32 = lane & 31;
  const int N = a.N;
  int b, hq, iq;
  map_q_block((N + BR - 1) / BR, a.B, a.Hq, a.Hkv, b, hq, iq);
  const int hkv = hq / (a.Hq / a.Hkv);
  const size_t qhead = (size_t)(b * a.Hq + hq) * (size_t)N;
  const size_t kvhead = (size_t)(b * a.Hkv + hkv) * (size_t)N;
  const unsigned char* Qg = (const unsigned char*)a.q + qhead * ROWB;
  const unsigned char* Kg = (const unsigned char*)a.k + kvhead * ROWB;
  const unsigned char* Vg = (const unsigned char*)a.v + kvhead * ROWB;
  const int q0 = iq * BR;
  const int qw = q0 + wave * 64;   // this wave's rows qw .. qw + 63, half f = rows qw + 32 f ..
  int myq[2];
  u32x4 qf[2][NS];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    myq[f] = qw + 32 * f + r32;
    if (myq[f] < N) {
      const unsigned char* qp = Qg + (size_t)myq[f] * ROWB + 16 * hh;
#pragma unroll
      for (int s = 0; s < NS; ++s) qf[f][s] = *(const u32x4*)(qp + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) qf[f][s] = u32x4{0, 0, 0, 0};
    }
  }
  unsigned char* const qpl = qpark + (wave * (NS - QP) * 64 + lane) * 16;
#pragma unroll
  for (int st = QP; st < NS; ++st) *(u32x4*)(qpl + (st - QP) * 1024) = qf[1][st];
  auto qop = [&](int f, int st) __attribute__((always_inline)) -> u32x4 {
    if (f == 1 && st >= QP) return *(const u32x4*)(qpl + (st - QP) * 1024);
    return qf[f][st];
  };
  const int nkv = (N + BC - 1) / BC;
  const int ntile = CAUSAL ? min(nkv, (min(q0 + BR, N) - 1) / BC + 1) : nkv;
  // keys some query of the wave sees: [0, uhi]; keys every query of half f sees: [0, whi[f]]
  const int uhi = qw >= N ? -1 : CAUSAL ? min(qw + 63, N - 1) : N - 1;
  int whi[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) whi[f] = CAUSAL ? min(qw + 32 * f, N - 1) : N - 1;
  int doff[IPW];
  Tiles::offsets(wave, lane, doff);
  const int ka = r32 * PK + 16 * hh;
  const int va = KBYTES + (4 * hh + ((lane & 15) >> 2)) * PV + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
  auto kread = [&](const unsigned char* sl, int h, int st) __attribute__((always_inline)) {
    return *(const u32x4*)(sl + h * 32 * PK + ka + 32 * st);
  };
  auto vread = [&](const unsigned char* sl, int hv, int h, int e) __attribute__((always_inline)) {
    const unsigned char* p = sl + (32 * hv + 16 * h) * PV;
    return cat(lds_read_tr(p + va + 64 * e), lds_read_tr(p + 8 * PV + va + 64 * e));
  };
  const float c2 = a.scale_log2;
  float mr[2] = {-FLT_MAX, -FLT_MAX}, l_run[2] = {0.f, 0.f};
  f32x16 o[2][NE];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[f][e][v] = 0.f;
  // S^T of half f for the keys of unit k0 (half h of slot sl), masked: -inf past the row's
  // position (causal) or past the end
  auto mask = [&](f32x16& x, int f, int k0) __attribute__((always_inline)) {
    if (!(k0 + 31 <= whi[f])) {
      int lim = N - k0 - 4 * hh;
      if (CAUSAL) lim = min(lim, myq[f] - k0 - 4 * hh + 1);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + (v & 3) >= lim) x[v] = -INFINITY;
    }
  };
  auto rowsum = [&](const f32x16& p) __attribute__((always_inline)) {
    float t[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) t[v] = p[2 * v] + p[2 * v + 1];
#pragma unroll
    for (int v = 0; v < 4; ++v) t[v] = t[2 * v] + t[2 * v + 1];
    return (t[0] + t[1]) + (t[2] + t[3]);
  };
  // unit u = keys 32u .. 32u+31, half h of the tile in slot sl
  auto unit = [&](int u, const unsigned char* sl, int h) __attribute__((always_inline)) {
    const int k0 = u * 32;
    if (k0 > uhi) return;   // wave-uniform: no query of this wave sees these keys
    // both halves' scores, each K operand read once for the two products
    f32x16 s[2];
    u32x4 kf = kread(sl, h, 0);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const u32x4 kc = kf;
      if (st + 1 < NS) kf = kread(sl, h, st + 1);
      s[0] = E::mma(kc, qf[0][st], st == 0 ? zero16() : s[0]);
      s[1] = E::mma(kc, qop(1, st), st == 0 ? zero16() : s[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P of both halves from the stale reference, in place of the scores (as in
    // fwd_unit_kernel: no row max on the common path)
    float rs[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      mask(s[f], f, k0);
#pragma unroll
      for (int v = 0; v < 16; ++v) s[f][v] = fast_exp2(fmaf(s[f][v], c2, -mr[f]));
      rs[f] = rowsum(s[f]);
    }
    const bool slow0 = __builtin_amdgcn_ballot_w64(!(rs[0] <= TAU_SUM)) != 0;
    const bool slow1 = __builtin_amdgcn_ballot_w64(!(rs[1] <= TAU_SUM)) != 0;
    if (slow0 || slow1) {
      // a half where some lane's P sums past TAU_SUM (or has no reference yet) takes the
      // slow path of fwd_unit_kernel on its scores formed again (the same products in the
      // same order, so the same bits; the registers do not keep the scores past the
      // exponentials): the row max, the reference raised to it (plus HEADROOM), O and
      // the row sum rescaled, P formed again
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        if (!(f == 0 ? slow0 : slow1)) continue;
        f32x16 x;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          x = E::mma(kread(sl, h, st), qop(f, st), st == 0 ? zero16() : x);
          __builtin_amdgcn_sched_barrier(0);   // one operand read at a time on this rare path
        }
        mask(x, f, k0);
        float mx = x[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, x[v]);
        const float mnew = fmaxf(mr[f], half_max(mx) * c2 + HEADROOM);
        const float alpha = fast_exp2(mr[f] - mnew);   // 0 from the sentinel, 1 if unmoved
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[f][e][v] *= alpha;
        l_run[f] *= alpha;
        mr[f] = mnew;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[f][v] = fast_exp2(fmaf(x[v], c2, -mr[f]));
        rs[f] = rowsum(s[f]);
      }
    }
    u32x4 pf[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      l_run[f] += rs[f];
      pf[f][0] = u32x4{E::pack(s[f][0], s[f][1]), E::pack(s[f][2], s[f][3]), E::pack(s[f][4], s[f][5]),
                       E::pack(s[f][6], s[f][7])};
      pf[f][1] = u32x4{E::pack(s[f][8], s[f][9]), E::pack(s[f][10], s[f][11]), E::pack(s[f][12], s[f][13]),
                       E::pack(s[f][14], s[f][15])};
    }
    // O^T += V^T P^T for both halves, each V operand read once for the two products
    u32x4 vf = vread(sl, h, 0, 0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < 2 * NE; ++k) {
      const int t = k / NE, e = k % NE;
      const u32x4 vc = vf;
      if (k + 1 < 2 * NE) vf = vread(sl, h, (k + 1) / NE, (k + 1) % NE);
      o[0][e] = E::mma(vc, pf[0][t], o[0][e]);
      o[1][e] = E::mma(vc, pf[1][t], o[1][e]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto dma = [&](int j, unsigned char* sl) __attribute__((always_inline)) {
    Tiles::load(Kg, Vg, N, j, wave, doff, sl);
  };
  auto tile = [&](auto Tc, int j) __attribute__((always_inline)) {
    constexpr int T = decltype(Tc)::value;
    unsigned char* const sc = slot(T);
    if (j > 0) {
      wait_loads();
      __syncthreads();
    }
    if (j + NSL - 1 < ntile) dma(j + NSL - 1, slot((T + NSL - 1) % NSL));
    unit(2 * j, sc, 0);
    unit(2 * j + 1, sc, 1);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  dma(0, slot0);
  if (ntile > 1) dma(1, slot1);
  wait_loads();
  __syncthreads();
  for (int j = 0; j < ntile; j += NSL) {
    tile(I0{}, j);
    if (j + 1 >= ntile) break;
    tile(I1{}, j + 1);
    if (j + 2 >= ntile) break;
    tile(I2{}, j + 2);
  }
  // the rows again from the lane number (mbcnt) and the wave's first row, so that no row
  // index has to stay live across the tile loop for these stores
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const float l_tot = half_sum(l_run[f]);
    const int row = qw + 32 * f + (lane_e & 31);
    if (row < N) {
      store_row16<E>((unsigned char*)a.o + (qhead + row) * ROWB, o[f], 1.f / l_tot, lane_e >> 5);
      if (lane_e < 32) a.lse[qhead + row] = (mr[f] + log2f(l_tot)) * kLn2;
    }
  }
}

// Waves per workgroup of fwd_unit_kernel.  d = 64: 8 (two workgroups per CU beat one
// of 16 at every measured shape).  d = 128: 12, one workgroup of 384 rows per CU; 6
// (192 rows, two per CU) when the 384-row grid is small — at most 128 workgroups, or
// 256 when causal, where a single long diagonal block would otherwise set the time.
// Past that the 6-wave grid loses: two workgroups per CU load every K/V tile twice.
// (Without key splits, the smallest grids take the key-split workgroups below.)
template <int D>
static int fwd_unit_waves(long long rows_blocks_of_384, bool causal) {
  if (D != 128) return 8;
  return rows_blocks_of_384 <= (causal ? 256 : 128) ? 6 : 12;
}

// d = 128 small grids, no key splits: 8 waves on 128 rows, two per 32 queries each taking
// one 32-key unit of every tile (KS = 2), while the 128-row grid fits the CUs once (256
// workgroups) or, causal, twice (its blocks differ in length).  A block's chain of units
// halves and its rows spread over more workgroups: 1.15-1.55x faster at one sequence of
// 1-8K tokens (16 heads of 1024 causal 29 -> 23 us, of 2048 50 -> 37 us, 4 heads of 8192
// causal 188 -> 119 us); on 768 or more blocks (384 non-causal) it was 8-27 % slower.
static bool fwd_small_grid_split(long long rows_blocks_of_128, bool causal) {
  return rows_blocks_of_128 <= (causal ? 512 : 256);
}
// d = 64 (where a CU holds more, smaller workgroups): 4 waves on 64 rows while the 64-row
// grid has at most 512 blocks, 6 waves on 96 rows for causal grids of up to 1024 such
// blocks, else the 8-wave grid (measured: 16 heads of 1024 causal 21.4 -> 16.2 us, of 4096
// causal 66.8 -> 51.0 us; 4 heads over one K/V head at 8192 causal 126 -> 87 us; past these
// limits 10-50 % slower).  0: no split.
static int fwd_small_grid_split_waves_d64(long long rows_blocks_of_64, bool causal) {
  if (rows_blocks_of_64 <= 512) return 4;
  if (causal && rows_blocks_of_64 <= 1024) return 6;
  return 0;
}

template <class Tag, int D, bool CAUSAL, bool GEN>
static hipError_t launch_fwd_unit(const FwdArgs& a, int nq, bool causal, hipStream_t stream) {
  const long long bh = (long long)a.B * a.Hq;
  const int ks = GEN ? a.ksplit : 1;   // key splits multiply the grid
  if constexpr (D == 128) {
    if (ks == 1 && fwd_small_grid_split(bh * ((nq + 127) / 128), causal)) {
      constexpr int NWS = 8, BRS = 32 * NWS / 2;
      const long long nb = bh * ((nq + BRS - 1) / BRS);
      if (nb <= 0) return hipSuccess;
      hipLaunchKernelGGL((fwd_unit_kernel<Tag, D, CAUSAL, NWS, GEN, 2>), dim3((unsigned)nb), dim3(NWS * 64), 0, stream,
                         a);
      return hipGetLastError();
    }
  } else {
    const int nws = ks == 1 ? fwd_small_grid_split_waves_d64(bh * ((nq + 63) / 64), causal) : 0;
    if (nws != 0) {
      const int brs = 16 * nws;
      const long long nb = bh * ((nq + brs - 1) / brs);
      if (nb <= 0) return hipSuccess;
      if (nws == 4)
        hipLaunchKernelGGL((fwd_unit_kernel<Tag, D, CAUSAL, 4, GEN, 2>), dim3((unsigned)nb), dim3(4 * 64), 0, stream, a);
      else
        hipLaunchKernelGGL((fwd_unit_kernel<Tag, D, CAUSAL, 6, GEN, 2>), dim3((unsigned)nb), dim3(6 * 64), 0, stream, a);
      return hipGetLastError();
    }
  }
  const int nw = fwd_unit_waves<D>(bh * ((nq + 383) / 384) * ks, causal);
  const int br = 32 * nw;
  const long long nb = bh * ((nq + br - 1) / br) * ks;
  if (nb <= 0) return hipSuccess;
  if constexpr (D == 128) {
    if (nw == 6)
      hipLaunchKernelGGL((fwd_unit_kernel<Tag, D, CAUSAL, 6, GEN>), dim3((unsigned)nb), dim3(6 * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_unit_kernel<Tag, D, CAUSAL, 12, GEN>), dim3((unsigned)nb), dim3(12 * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fwd_unit_kernel<Tag, D, CAUSAL, 8, GEN>), dim3((unsigned)nb), dim3(8 * 64), 0, stream, a);
  }
  return hipGetLastError();
}

// fa_fwd: at d = 128 the 64-query waves (512-row workgroups, one per CU) once their grid
// fills the CUs at least twice when causal (the blocks differ in length) or once when
// not (2-3 % faster causal, 8-10 % not, at N = 8192-16384); smaller grids keep the 32-query
// kernel, whose smaller workgroups spread the work over more CUs.
template <class Tag, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  if constexpr (D == 128) {
    constexpr int NW2 = 8;
    const long long nb = (long long)a.B * a.Hq * ((a.N + 64 * NW2 - 1) / (64 * NW2));
    if (nb >= (CAUSAL ? 512 : 256)) {
      hipLaunchKernelGGL((fwd_unit2_kernel<Tag, D, CAUSAL, NW2>), dim3((unsigned)nb), dim3(NW2 * 64), 0, stream, a);
      return hipGetLastError();
    }
  }
  return launch_fwd_unit<Tag, D, CAUSAL, false>(a, a.N, CAUSAL, stream);
}

template <class Tag, int D>
static hipError_t launch_fwd_masked_t(const FwdArgs& a, hipStream_t stream) {
  if (a.bidx == nullptr)   // no block lists: the unit kernel in its general mode
    return launch_fwd_unit<Tag, D, false, true>(a, a.maxq, a.wr >= 0, stream);
  // block lists name 256-query blocks: the 8-wave kernel
  constexpr int BR = 256;
  const int nqb = (a.maxq + BR - 1) / BR;
  const long long nblocks = (long long)a.B * a.Hq * nqb;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<Tag, D, false, true>), dim3((unsigned)nblocks), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_masked(const FwdArgs& a, int d, bool bf16, hipStream_t stream) {
  if (bf16) return d == 128 ? launch_fwd_masked_t<bf16_tag, 128>(a, stream) : launch_fwd_masked_t<bf16_tag, 64>(a, stream);
  return d == 128 ? launch_fwd_masked_t<f16_tag, 128>(a, stream) : launch_fwd_masked_t<f16_tag, 64>(a, stream);
}

hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16, bool causal, hipStream_t stream) {
#define FA_FWD_CASE(TAG, D) \
  return causal ? launch_fwd_t<TAG, D, true>(a, stream) : launch_fwd_t<TAG, D, false>(a, stream)
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
