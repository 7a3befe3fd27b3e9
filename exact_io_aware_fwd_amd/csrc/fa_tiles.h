// Tile movement and work mapping shared by the query-block-outer kernels (the
// forward pass and the dQ pass of the backward): 64-row tiles of two [N, d]
// tensors of one head go from HBM straight into LDS, and block ids are mapped to
// (batch, head, query block).
#pragma once

#include "fa_device.h"

namespace fa {

typedef __attribute__((address_space(3))) void lvoid;

// XOR on the 16-byte chunk index of row r of a tile that is read both by rows (16
// bytes per lane, 16 consecutive rows) and transposed (ds_read_b64_tr_b16, 8 bytes per
// lane from 4 consecutive rows): with unpadded rows both patterns then hit distinct
// banks (measured free of bank conflicts), and each address is a lane constant XOR an
// instruction constant.  CH = 16-byte chunks per row.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

// Per-lane LDS offsets into a swizzled tile (rows of ROWB bytes, CH = ROWB/16 chunks).
//  rows(st):  the A operand of a 32x32x16 MFMA from rows r32, chunk 2st + hh
//             -> rows_a0 ^ (st << 5)
//  tr(e, u):  the A operand of a transposed product from rows 16t + 8u + R,
//             elements 32e + 16x + 4y (ds_read_b64_tr_b16)
//             -> (16t + 8u) * ROWB + (tr_lane ^ tr_inst(e, u))
template <int ROWB>
struct SwzOffsets {
  static constexpr int CH = ROWB / 16;
  static __device__ __forceinline__ int rows_a0(int lane) {
    const int hh = lane >> 5, r32 = lane & 31;
    return r32 * ROWB + ((hh ^ swz<CH>(r32)) << 4);
  }
  static __device__ __forceinline__ int tr_lane(int lane) {
    const int hh = lane >> 5, R = 4 * hh + ((lane & 15) >> 2), x = (lane >> 4) & 1, y = lane & 3;
    int lp;
    if constexpr (CH == 16) lp = (2 * x) ^ (y >> 1) ^ ((R & 3) << 2) ^ hh;
    else lp = (2 * x) ^ (y >> 1) ^ (((R >> 1) & 3) << 1);
    return R * ROWB + (lp << 4) + 8 * (y & 1);
  }
  static constexpr int tr_inst(int e, int u) { return (CH == 16 ? ((4 * e) ^ (2 * u)) : ((4 * e) ^ u)) << 4; }
};

// A pair of 64-row tiles (tensor A then tensor B) in one LDS slot, rows padded to
// pitches PA and PB bytes, or, with SWZ_A (SWZ_B), tensor A (B) unpadded with its chunks
// swizzled as above.  With the 64 four-byte banks of the CDNA4 LDS:
//   pitch row+16 B: 16 lanes reading 16 bytes from 16 consecutive rows hit distinct banks;
//   pitch row+64 B: 32 lanes reading 8 bytes from 4 consecutive rows (ds_read_b64_tr_b16)
//                   hit distinct banks.
// Both were measured free of bank conflicts.  The slot is filled by wave-wide
// 16-byte-per-lane loads: load n (n = wave + NW*i) covers slot bytes [1024n, 1024n+1024).
template <int ROWB, int PA, int PB, int NW, bool SWZ_A = false, bool SWZ_B = false>
struct TilePair {
  static constexpr int ABYTES = 64 * PA;
  static constexpr int BBYTES = 64 * PB;
  static constexpr int SLOT = ABYTES + BBYTES;
  static constexpr int AI = ABYTES / 1024;          // loads per A tile
  static constexpr int NI = AI + BBYTES / 1024;     // loads per slot
  static constexpr int IPW = (NI + NW - 1) / NW;    // loads per wave per slot
  static_assert(ABYTES % 1024 == 0 && BBYTES % 1024 == 0, "tiles are whole wave loads");

  // Byte of the tile's rows that this lane's 16 bytes of load i come from.  Lanes
  // landing on row padding re-fetch byte 0 (any valid address will do).
  static_assert(!SWZ_A || PA == ROWB, "a swizzled tile is unpadded");
  static_assert(!SWZ_B || PB == ROWB, "a swizzled tile is unpadded");
  static __device__ __forceinline__ void offsets(int wave, int lane, int* doff) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int n = wave + NW * i;
      const int P = n < AI ? PA : PB;
      const int o = (n < AI ? n : n - AI) * 1024 + lane * 16;
      const int row = o / P, col = o - (o / P) * P;
      if ((SWZ_A && n < AI) || (SWZ_B && n >= AI))
        doff[i] = row * ROWB + (((col >> 4) ^ swz<ROWB / 16>(row)) << 4);
      else
        doff[i] = col < ROWB ? row * ROWB + col : 0;
    }
  }

  // Tile t (rows 64t .. 64t+63) of A and B into slot `slot`.  The loads go through
  // buffer descriptors whose range ends at row N, so rows past the end arrive as zeros.
  static __device__ __forceinline__ void load(const unsigned char* Ag, const unsigned char* Bg, int N, int t,
                                              int wave, const int* doff, unsigned char* slotp) {
    const int kb = t * 64;
    const int bytes = (N - kb) * ROWB;
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Ag + (size_t)kb * ROWB), (short)0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t br =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Bg + (size_t)kb * ROWB), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int n = wave + NW * i;
      if (n < AI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lvoid*)(slotp + n * 1024), 16, doff[i], 0, 0, 0);
      else if (n < NI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lvoid*)(slotp + n * 1024), 16, doff[i], 0, 0, 0);
    }
  }
};

// Block id -> (batch, query head, query block) for kernels with one workgroup per
// query block.  Blocks are dealt round-robin to the 8 XCDs; when the number of
// (batch, kv-head) groups is a multiple of 8, XCD x serves groups x, x+8, ... so
// their K/V stay in that XCD's L2.  Within an XCD, slots run over query blocks
// from the last (longest when causal) down.
__device__ __forceinline__ void map_q_block(int nqb, int B, int Hq, int Hkv, int& b, int& hq, int& iq, int bid) {
  const int G = Hq / Hkv;
  const int ngroups = B * Hkv;
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
__device__ __forceinline__ void map_q_block(int nqb, int B, int Hq, int Hkv, int& b, int& hq, int& iq) {
  map_q_block(nqb, B, Hq, Hkv, b, hq, iq, (int)blockIdx.x);
}

}  // namespace fa
