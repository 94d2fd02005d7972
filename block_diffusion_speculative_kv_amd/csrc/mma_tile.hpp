// LDS-tiled bf16 MFMA main loop shared by the dense projections with many
// rows and by the LM head at batch scale.
//
// A workgroup of 4 waves (2 x 2) computes a BN x BM block of C = W . X^T,
// W [N, K] the weight (MFMA A operand, output features), X [M, K] the
// activations (MFMA B operand, rows); each wave owns NW x MW 16x16 tiles.
// k advances in stages of 64: every thread copies NW + MW 16-byte vectors of
// the next stage from global memory into registers while the waves multiply
// the current stage out of LDS, then writes them to the other LDS buffer;
// one barrier per stage.  LDS rows are padded by 16 bytes (row stride 144 B),
// so the 16 rows one fragment read touches fall on distinct banks.
//
// PERM: inside each pair of vocabulary tiles, A-operand row 4q + e of tile
// 2p + s is output feature 32p + 8q + 4s + e, so lane group g ends up with
// the 8 consecutive features 32p + 8g .. 32p + 8g + 7 (one Philox block in
// the LM head's sampling epilogue).
#pragma once

#include "common.hpp"

namespace dstill {

constexpr int TK = 64;       // k per LDS stage
constexpr int TKP = TK + 8;  // padded LDS row (elements)

template <int NW, int MW>
struct TileSmem {
  static constexpr int BN = 32 * NW, BM = 32 * MW;
  bf16 w[2][BN * TKP];
  bf16 x[2][BM * TKP];
};

// One stage of a workgroup's W and X tiles held in registers.
template <int NW, int MW>
struct TileRegs {
  bf16x8 w[NW], x[MW];
};

// Global -> register -> LDS copier for one workgroup's W and X tiles.  Each
// matrix is addressed from one wave-uniform base (the block's first row,
// advanced by whole stages) plus a 32-bit per-thread element offset, which
// keeps the per-thread address state small.
template <int NW, int MW>
struct TileLoader {
  static constexpr int BN = 32 * NW, BM = 32 * MW;
  const bf16 *wbase, *xbase;
  int woff[NW], xoff[MW];

  // wrow(i) / xrow(i): element offset of tile row i from wb / xb (already
  // clamped to a valid row; must fit in 31 bits); k0: first k of this
  // workgroup's range.
  template <typename WRow, typename XRow>
  __device__ __forceinline__ void init(const bf16 *wb, WRow wrow, const bf16 *xb, XRow xrow,
                                       long k0) {
    wbase = wb + k0;
    xbase = xb + k0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int idx = threadIdx.x + 256 * i;
      woff[i] = wrow(idx >> 3) + (idx & 7) * 8;
    }
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int idx = threadIdx.x + 256 * i;
      xoff[i] = xrow(idx >> 3) + (idx & 7) * 8;
    }
  }
  __device__ __forceinline__ void load(TileRegs<NW, MW> &r, int stage) const {
    const bf16 *wb = wbase + (long)stage * TK;
    const bf16 *xb = xbase + (long)stage * TK;
#pragma unroll
    for (int i = 0; i < NW; ++i) r.w[i] = *reinterpret_cast<const bf16x8 *>(wb + woff[i]);
#pragma unroll
    for (int i = 0; i < MW; ++i) r.x[i] = *reinterpret_cast<const bf16x8 *>(xb + xoff[i]);
  }
  __device__ __forceinline__ void store(TileSmem<NW, MW> &sm, int buf,
                                        const TileRegs<NW, MW> &r) const {
    const int base = (threadIdx.x >> 3) * TKP + (threadIdx.x & 7) * 8;
#pragma unroll
    for (int i = 0; i < NW; ++i)
      *reinterpret_cast<bf16x8 *>(&sm.w[buf][base + 32 * TKP * i]) = r.w[i];
#pragma unroll
    for (int i = 0; i < MW; ++i)
      *reinterpret_cast<bf16x8 *>(&sm.x[buf][base + 32 * TKP * i]) = r.x[i];
  }
};

// Row (within the workgroup's BN rows) that lane r16 feeds for tile i.
template <int NW, bool PERM>
__device__ __forceinline__ int tile_a_row(int wn, int i, int r16) {
  if (PERM) return wn * 16 * NW + 32 * (i >> 1) + 8 * (r16 >> 2) + 4 * (i & 1) + (r16 & 3);
  return wn * 16 * NW + 16 * i + r16;
}

template <int NW, int MW, bool PERM>
__device__ __forceinline__ void tile_mainloop(TileSmem<NW, MW> &sm, TileLoader<NW, MW> &ld,
                                              int nst, f32x4 (&acc)[NW][MW]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wn = wave & 1, wm = wave >> 1;
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int j = 0; j < MW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nst <= 0) return;
  int arow[NW], brow[MW];
#pragma unroll
  for (int i = 0; i < NW; ++i) arow[i] = tile_a_row<NW, PERM>(wn, i, r16) * TKP + 8 * g;
#pragma unroll
  for (int j = 0; j < MW; ++j) brow[j] = (wm * 16 * MW + 16 * j + r16) * TKP + 8 * g;

  auto compute = [&](int cur) {
    const bf16 *ws = sm.w[cur];
    const bf16 *xs = sm.x[cur];
#pragma unroll
    for (int kk = 0; kk < TK / 32; ++kk) {
      bf16x8 a[NW], b[MW];
#pragma unroll
      for (int i = 0; i < NW; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(ws + arow[i] + 32 * kk);
#pragma unroll
      for (int j = 0; j < MW; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(xs + brow[j] + 32 * kk);
#pragma unroll
      for (int i = 0; i < NW; ++i)
#pragma unroll
        for (int j = 0; j < MW; ++j) acc[i][j] = Mma<bf16>::run(a[i], b[j], acc[i][j]);
    }
  };
  // stage s lives in LDS buffer s & 1; the next stage waits in registers
  TileRegs<NW, MW> r;
  ld.load(r, 0);
  ld.store(sm, 0, r);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int cur = s & 1;
    if (s + 1 < nst) ld.load(r, s + 1);
    compute(cur);
    if (s + 1 < nst) ld.store(sm, cur ^ 1, r);
    __syncthreads();
  }
}

// XCD-aware placement: workgroup L runs on XCD L mod 8.  The m-blocks of one
// n-block get consecutive slots on the same XCD, so they stream the same
// weight tile through one L2 at about the same time.
__device__ __forceinline__ void xcd_block(int L, int nmb, int *nb, int *mb) {
  const int xcd = L & 7, slot = L >> 3;
  *nb = (slot / nmb) * 8 + xcd;
  *mb = slot % nmb;
}

}  // namespace dstill
