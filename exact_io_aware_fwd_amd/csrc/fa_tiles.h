// Tile movement and work mapping shared by the query-block-outer kernels (the
// forward pass and the dQ pass of the backward): 64-row tiles of two [N, d]
// tensors of one head go from HBM straight into LDS, and block ids are mapped to
// (batch, head, query block).
#pragma once

#include "fa_device.h"

namespace fa {

typedef __attribute__((address_space(3))) void lvoid;

// A pair of 64-row tiles (tensor A then tensor B) in one LDS slot, rows padded to
// pitches PA and PB bytes.  With the 64 four-byte banks of the CDNA4 LDS:
//   pitch row+16 B: 16 lanes reading 16 bytes from 16 consecutive rows hit distinct banks;
//   pitch row+64 B: 32 lanes reading 8 bytes from 4 consecutive rows (ds_read_b64_tr_b16)
//                   hit distinct banks.
// Both were measured free of bank conflicts.  The slot is filled by wave-wide
// 16-byte-per-lane loads: load n (n = wave + NW*i) covers slot bytes [1024n, 1024n+1024).
template <int ROWB, int PA, int PB, int NW>
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
  static __device__ __forceinline__ void offsets(int wave, int lane, int* doff) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int n = wave + NW * i;
      const int P = n < AI ? PA : PB;
      const int o = (n < AI ? n : n - AI) * 1024 + lane * 16;
      const int row = o / P, col = o - (o / P) * P;
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
__device__ __forceinline__ void map_q_block(int nqb, int B, int Hq, int Hkv, int& b, int& hq, int& iq) {
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

}  // namespace fa
