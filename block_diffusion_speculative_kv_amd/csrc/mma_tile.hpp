// LDS-tiled bf16 MFMA main loop shared by the dense projections with many
// rows and by the LM head at batch scale.
//
// A workgroup of WN x WM waves computes a BN x BM block of C = W . X^T,
// W [N, K] the weight (MFMA A operand, output features), X [M, K] the
// activations (MFMA B operand, rows); each wave owns NW x MW 16x16 tiles.
// k advances in stages of KT through rings of LDS buffers filled by direct
// global->LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land at
// the instruction's LDS base + 16 * lane), issued ahead of the multiply: the
// copies need no registers and no LDS write instructions, and the only wait
// is one vmcnt + barrier per stage.  The loads are issued from inline
// assembly with an explicit vmcnt, because the compiler, which cannot tell
// the ring buffers apart, would otherwise wait for every outstanding copy
// before each LDS read.
//
// LDS rows are KT * 2 bytes (unpadded); 16-byte chunk c of row r sits at
// chunk c ^ tile_swz(r), so the 16 rows of one fragment read (contiguous
// rows, or the permuted rows below) fall on 16 distinct bank groups.
//
// PERM: inside each pair of vocabulary tiles, A-operand row 4q + e of tile
// 2p + s is output feature 32p + 8q + 4s + e, so lane group g ends up with
// the 8 consecutive features 32p + 8g .. 32p + 8g + 7 (one Philox block in
// the LM head's sampling epilogue).
#pragma once

#include <cstdint>

#include "common.hpp"
#include "dma.hpp"

namespace dstill {

// Chunk swizzle.  KT = 64 (8 chunks, 2 rows per 256-byte bank window): bits
// (r1, r3, r2 ^ r4); KT = 32 (4 chunks, 4 rows per window): bits (r2 ^ r4,
// r3).  Over 16 contiguous rows (r0..r3 vary) and over the permuted rows of
// one tile (r0, r1, r3, r4 vary) the 16-byte slot of a given logical chunk
// within its bank window takes 16 distinct values.
template <int KT>
__device__ __forceinline__ int tile_swz(int r) {
  if (KT == 64) return ((r >> 1) & 1) | ((r >> 2) & 2) | ((((r >> 2) ^ (r >> 4)) & 1) << 2);
  return (((r >> 2) ^ (r >> 4)) & 1) | ((r >> 2) & 2);
}

// Byte offset of lane (g, r16)'s 16-byte k-chunk 4 kk + g of LDS row r.
template <int KT>
__device__ __forceinline__ int tile_frag_off(int r, int kk, int g) {
  return r * (KT * 2) + (((4 * kk + g) ^ tile_swz<KT>(r)) * 16);
}

// One tile configuration: WN x WM waves, each owning NW x MW 16x16 output
// tiles, so a workgroup computes BN = 16 NW WN output features x BM = 16 MW
// WM rows.  KT: k per LDS stage (64 or 32).  W stages sit in a ring of NSW
// buffers, X stages in a ring of NSX: the weight, streamed once from HBM, is
// fetched NSW - 1 stages ahead of the multiply, the activations (re-read by
// every weight block, mostly from L2) NSX - 1 stages ahead.  A row of a stage
// is KT * 2 bytes, CPR = KT / 8 chunks of 16 bytes; one copy instruction (64
// lanes x 16 bytes) fills RPI = 1024 / (KT * 2) rows.
//
// 2 x 2 waves with 128 x 128 tiles keep two workgroups on a compute unit;
// 2 x 4 waves with 256 x 256 tiles take one compute unit each and halve the
// bytes copied into LDS per product term, which is what bounds the smaller
// tile once the rows are many.
template <int WN_, int WM_, int NW_, int MW_, int KT_, int NSW_, int NSX_>
struct TileEngine {
  static constexpr int WN = WN_, WM = WM_, NW = NW_, MW = MW_, KT = KT_, NSW = NSW_, NSX = NSX_;
  static constexpr int NWAVES = WN * WM, NT = 64 * NWAVES;
  static constexpr int BN = 16 * NW * WN, BM = 16 * MW * WM;
  static constexpr int CPR = KT / 8, RPI = 64 / CPR;
  // copies per stage (TW, TX) and per wave (NCW, NCX): every wave takes the
  // same number of W copies; X copies may fall short by one on the last waves
  static constexpr int TW = BN / RPI, TX = BM / RPI;
  static constexpr int NCW = TW / NWAVES, NCX = (TX + NWAVES - 1) / NWAVES;
  static_assert(KT == 64 || KT == 32, "stage depth");
  static_assert(NSX == 2 && NSW >= 3 && NSW <= 8, "ring depths");
  static_assert(NCW * (NSW - 2) < 64, "vmcnt holds the copies left in flight");
  static_assert(TW * RPI == BN && TX * RPI == BM && NCW * NWAVES == TW, "whole copies");

  struct Smem {
    bf16 w[NSW][BN * KT];
    bf16 x[NSX][BM * KT];
  };

  // Copier for one workgroup's W and X tiles.  Copy i of wave w fills row
  // group NWAVES i + w (RPI rows; X copies only while the group exists), lane
  // L loading row RPI * group + L / CPR, logical chunk (L % CPR) ^
  // tile_swz(row).  A wave's X copies are issued before any W copy the wait
  // may leave in flight, so one issuing fewer of them waits no less.  Each matrix is addressed from
  // one wave-uniform base (the block's first row, advanced by whole stages)
  // plus a 32-bit per-lane byte offset.
  struct Loader {
    const char *wbase, *xbase;
    uint32_t woff[NCW], xoff[NCX];

    // wrow(r) / xrow(r): element offset of tile row r from wb / xb (already
    // clamped to a valid row; twice it must fit in 32 bits); k0: first k of
    // this workgroup's range.
    template <typename WRow, typename XRow>
    __device__ __forceinline__ void init(const bf16 *wb, WRow wrow, const bf16 *xb, XRow xrow,
                                         long k0) {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      wbase = reinterpret_cast<const char *>(wb + k0);
      xbase = reinterpret_cast<const char *>(xb + k0);
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        const int r = RPI * (NWAVES * i + wave) + lane / CPR;
        woff[i] = (uint32_t)wrow(r) * 2u + (uint32_t)(((lane % CPR) ^ tile_swz<KT>(r)) * 16);
      }
#pragma unroll
      for (int i = 0; i < NCX; ++i) {
        const int r = min(RPI * (NWAVES * i + wave) + lane / CPR, BM - 1);
        xoff[i] = (uint32_t)xrow(r) * 2u + (uint32_t)(((lane % CPR) ^ tile_swz<KT>(r)) * 16);
      }
    }
    __device__ __forceinline__ void issue_w(Smem &sm, int stage) const {
      const char *wb = wbase + (long)stage * KT * 2;
      const uint32_t wl = lds_u32(&sm.w[stage % NSW][0]) + (threadIdx.x >> 6) * 1024;
#pragma unroll
      for (int i = 0; i < NCW; ++i) dma16(wb, woff[i], wl + i * 1024 * NWAVES);
    }
    // Copy i (compile-time) of this wave for one stage.
    __device__ __forceinline__ void issue_w_one(Smem &sm, int stage, int i) const {
      const char *wb = wbase + (long)stage * KT * 2;
      const uint32_t wl = lds_u32(&sm.w[stage % NSW][0]) + (threadIdx.x >> 6) * 1024;
      dma16(wb, woff[i], wl + i * 1024 * NWAVES);
    }
    __device__ __forceinline__ void issue_x_one(Smem &sm, int stage, int i) const {
      const char *xb = xbase + (long)stage * KT * 2;
      const uint32_t xl = lds_u32(&sm.x[stage % NSX][0]) + (threadIdx.x >> 6) * 1024;
      if (TX % NWAVES == 0 || NWAVES * i + (int)(threadIdx.x >> 6) < TX)
        dma16(xb, xoff[i], xl + i * 1024 * NWAVES);
    }
    __device__ __forceinline__ void issue_x(Smem &sm, int stage) const {
      const char *xb = xbase + (long)stage * KT * 2;
      const uint32_t xl = lds_u32(&sm.x[stage % NSX][0]) + (threadIdx.x >> 6) * 1024;
#pragma unroll
      for (int i = 0; i < NCX; ++i)
        if (TX % NWAVES == 0 || NWAVES * i + (int)(threadIdx.x >> 6) < TX)
          dma16(xb, xoff[i], xl + i * 1024 * NWAVES);
    }
  };

  // Row (within the workgroup's BN rows) that lane r16 of wave column wn feeds
  // for tile i.  PERM: inside each pair of tiles, A-operand row 4q + e of tile
  // 2p + s is feature 32p + 8q + 4s + e of the wave's band.
  template <bool PERM>
  __device__ __forceinline__ static int a_row(int wn, int i, int r16) {
    if (PERM) return wn * 16 * NW + 32 * (i >> 1) + 8 * (r16 >> 2) + 4 * (i & 1) + (r16 & 3);
    return wn * 16 * NW + 16 * i + r16;
  }

  template <bool PERM>
  __device__ __forceinline__ static void mainloop(Smem &sm, const Loader &ld, int nst,
                                                  f32x4 (&acc)[NW][MW]) {
    constexpr int NKK = KT / 32;
    static_assert(NKK == 2, "two 32-deep k-steps per stage");
    static_assert(!PERM || NW % 2 == 0, "permuted rows pair the tiles");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int wn = wave % WN, wm = wave / WN;
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int j = 0; j < MW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nst <= 0) return;
    int aoff[NW][NKK], boff[MW][NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int i = 0; i < NW; ++i) aoff[i][kk] = tile_frag_off<KT>(a_row<PERM>(wn, i, r16), kk, g);
#pragma unroll
      for (int j = 0; j < MW; ++j)
        boff[j][kk] = tile_frag_off<KT>(wm * 16 * MW + 16 * j + r16, kk, g);
    }
    // Fragments of one k-step: the second k-step of stage s is read while the
    // first k-step's products run, and the first k-step of stage s + 1 is
    // read (after the barrier that publishes its copies) while the second
    // k-step's products run, so the matrix pipe never waits for LDS after a
    // barrier.  Once every wave has read both k-steps of stage s, its
    // buffers are free: the barrier in the middle of stage s lets the copies
    // of stage s + 2 (activations) refill them, and the weight copies of
    // stage s + NSW - 1 go into the buffer freed by the previous barrier,
    // during the first half of stage s.
    //
    // Copies are spread between groups of products rather than issued in one
    // burst after the barrier, so no wave holds its products back behind a
    // run of copy instructions (faster on the short per-cycle products, no
    // slower on the long ones).  Each half stage is cut into as many groups
    // as it has copies (a copy, then its share of the fragment reads and of
    // the products), fenced by scheduling barriers so the compiler keeps that
    // order.
    bf16x8 fa[2][NW], fb[2][MW];
    auto read = [&](int s, int kk, int set) {
      const char *ws = reinterpret_cast<const char *>(&sm.w[s % NSW][0]);
      const char *xs = reinterpret_cast<const char *>(&sm.x[s % NSX][0]);
#pragma unroll
      for (int i = 0; i < NW; ++i) fa[set][i] = *reinterpret_cast<const bf16x8 *>(ws + aoff[i][kk]);
#pragma unroll
      for (int j = 0; j < MW; ++j) fb[set][j] = *reinterpret_cast<const bf16x8 *>(xs + boff[j][kk]);
    };
    // Half stage: products of fragment set `set`; reads of the other set from
    // stage rs, k-step rkk; copies copy(c) for c < NC.
    auto half = [&](auto set_c, int rs, auto rkk_c, auto nc_c, auto copy) {
      constexpr int set = decltype(set_c)::value, oset = set ^ 1, rkk = decltype(rkk_c)::value;
      constexpr int NC = decltype(nc_c)::value, NG = NC > 0 ? NC : 1;
      constexpr int NP = NW * MW, NF = NW + MW;
      const char *ws = reinterpret_cast<const char *>(&sm.w[rs % NSW][0]);
      const char *xs = reinterpret_cast<const char *>(&sm.x[rs % NSX][0]);
      static_for<NG>([&](auto G) {
        constexpr int q = decltype(G)::value;
        constexpr int f0 = q * NF / NG, f1 = (q + 1) * NF / NG;
        constexpr int p0 = q * NP / NG, p1 = (q + 1) * NP / NG;
        if constexpr (NC > 0) copy(G);
        static_for<f1 - f0>([&](auto F) {
          constexpr int f = f0 + decltype(F)::value;
          if constexpr (f < NW)
            fa[oset][f] = *reinterpret_cast<const bf16x8 *>(ws + aoff[f][rkk]);
          else
            fb[oset][f - NW] = *reinterpret_cast<const bf16x8 *>(xs + boff[f - NW][rkk]);
        });
        static_for<p1 - p0>([&](auto P) {
          constexpr int p = p0 + decltype(P)::value, i = p / MW, j = p % MW;
          acc[i][j] = Mma<bf16>::run(fa[set][i], fb[set][j], acc[i][j]);
        });
        // reads and products alternate inside the group
        constexpr int nf = f1 - f0, np = p1 - p0;
        constexpr int ratio = nf > 0 && np / nf > 0 ? np / nf : 1;
        constexpr int inter = nf * ratio <= np ? nf : np / ratio;
        static_for<inter>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, ratio, 0);
        });
        if constexpr (nf > inter) __builtin_amdgcn_sched_group_barrier(0x100, nf - inter, 0);
        if constexpr (np > inter * ratio)
          __builtin_amdgcn_sched_group_barrier(0x008, np - inter * ratio, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // Issue order: W0, X0, W1 .. W(NSW - 2) before stage 0, then X1 after
    // the barrier that publishes stage 0.  In stage s: W(s + NSW - 1) in the
    // first half; after the barrier that publishes stage s + 1, X(s + 2).
    // The wait for stage s + 1 then leaves in flight only W(s + NSW - 1) if
    // it exists (W(s + 1) was issued before X(s + 1)).
    ld.issue_w(sm, 0);
    ld.issue_x(sm, 0);
#pragma unroll
    for (int p = 1; p <= NSW - 2; ++p)
      if (p < nst) ld.issue_w(sm, p);
    {
      const int later = min(NSW - 2, nst - 1);
      if (later == 0) {
        wait_vmcnt<0>();
      } else if (later == 1) {
        wait_vmcnt<NCW>();
      } else {
        static_for<(NSW > 3 ? NSW - 3 : 0)>([&](auto L) {
          constexpr int n = decltype(L)::value + 2;
          if (later == n) wait_vmcnt<n * NCW>();
        });
      }
    }
    __syncthreads();
    if (1 < nst) ld.issue_x(sm, 1);
    read(0, 0, 0);
    for (int s = 0; s < nst; ++s) {
      // first half: products of k-step 0, reads of k-step 1, weight copies
      {
        const int ws_ = s + NSW - 1;
        const bool cw = ws_ < nst;
        half(I0{}, s, I1{}, std::integral_constant<int, NCW>{}, [&](auto C) {
          if (cw) ld.issue_w_one(sm, ws_, decltype(C)::value);
        });
      }
      if (s + 1 < nst) {
        if (s + NSW - 1 < nst) wait_vmcnt<NCW>();
        else wait_vmcnt<0>();
        __syncthreads();
      }
      // second half: products of k-step 1, reads of stage s + 1's k-step 0
      // (the last stage re-reads its own: unused, harmless), activation
      // copies
      const bool cx = s + 2 < nst;
      const int xs_ = s + 2;
      half(I1{}, min(s + 1, nst - 1), I0{}, std::integral_constant<int, NCX>{}, [&](auto C) {
        if (cx) ld.issue_x_one(sm, xs_, decltype(C)::value);
      });
    }
    __syncthreads();  // every wave is done with the rings: the caller may reuse them
  }
};

// XCD-aware placement: workgroup L runs on XCD L mod 8, which takes every
// eighth n-block (nn of them).  Within an XCD, slots go in groups of up to
// 8 m-blocks x all its n-blocks, m fastest: the workgroups that run together
// on one XCD cover at most 8 m-blocks and a few n-blocks, so both the weight
// tiles and the activation tiles they stream are shared through that XCD's
// L2.  With up to 8 m-blocks (every draft shape and the LM head) this is
// simply all m-blocks of one n-block in consecutive slots.
__device__ __forceinline__ void xcd_block(int L, int nmb, int nn, int *nb, int *mb) {
  constexpr int GM = 8;
  const int xcd = L & 7, s = L >> 3;
  const int per_group = GM * nn;
  const int first = (s / per_group) * GM;
  const int gsz = min(nmb - first, GM);
  const int r = s % per_group;
  *mb = first + r % gsz;
  *nb = (r / gsz) * 8 + xcd;
}

}  // namespace dstill
