// Shared LM head with a fused vocabulary-wide reduction (DStill, Experimental
// Setup and DFlash review, Training: the drafter reuses the target's frozen
// LM head; DStill, Inference: greedy top-1 or a sampled proposal per
// position; SPOT, Method: one Gumbel table shared per block slot).
//
// z = hidden . W^T is computed tile by tile on the matrix cores and reduced
// on the spot: per row and vocabulary block the kernel keeps the best score
// (z, or z/T + g for Gumbel-max sampling), its id (lowest id on ties), the
// runner-up score, z at the best id, max z, and the softmax mass at
// temperature T relative to the block's max.  The logits themselves are
// written only when the caller asks for them (rejection sampling needs the
// draft rows).  A second kernel merges the per-block records of each row in
// a fixed order, so results are deterministic.
//
// Layout: the weight is the MFMA A operand (16 vocabulary rows per tile) and
// the hidden rows the B operand.  Vocabulary rows inside each pair of tiles
// are permuted so that lane group g of a wave holds the 8 consecutive ids
// 8g .. 8g+7 of a 32-id span: exactly one Philox4x64-10 block.
//
// Main loops (bf16): up to 64 rows the weight streams once through an LDS
// ring of direct copies (HBM-bound); with more rows the tile engine of
// mma_tile.hpp re-uses each staged weight tile across 160 or 256 rows.  fp32
// (and shapes neither takes) load fragments straight into registers.  All
// end in the same per-lane reduction epilogue.
//
// Launch: the row blocks of one vocabulary block are placed on the same XCD
// (workgroup i runs on XCD i mod 8) and next to each other in dispatch order,
// so when there are several row blocks they read the weight tile through the
// same L2 at about the same time instead of fetching it again from HBM.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "dma.hpp"
#include "mma_tile.hpp"

namespace dstill {

constexpr int HEAD_VB = 256;  // vocabulary ids per workgroup, register path (64 per wave)
constexpr int HEAD_KT = 64;   // LDS path: k per stage
// LDS-path tiles (vocabulary ids x rows): 64 x 32 and 64 x 64 up to 64 rows
// when the streaming kernel does not take them (depth not a multiple of 128),
// 128 x 160 up to 160 rows (2 x 2 waves, two workgroups per CU; the 160-row
// tile with a two-deep weight ring to fit); 256 x 256 beyond (2 x 4 waves, one
// workgroup per CU, the weight three stages ahead in all of LDS), which
// copies half the bytes into LDS per product term.
template <int NW, int MW>
using HeadTile = TileEngine<2, 2, NW, MW, HEAD_KT, 3, 2>;
using HeadBigTile = TileEngine<2, 4, 8, 4, HEAD_KT, 3, 2>;
constexpr int NXCD = 8;

// Smallest vocabulary block of any path: sizes the partial-record workspace.
int head_vocab_block() { return 64; }  // the smallest block any path uses

struct RowStat {
  ArgTop2 arg;
  float zbest, zmax, m, s;
};

// Branch-free: a side with m = -inf (no ids) has s = 0 and weight 0, the
// other keeps its s exactly (expf(0) = 1), as a branch on -inf would.
__device__ __forceinline__ void ms_merge(float &m, float &s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  const float w1 = m == -INFINITY ? 0.f : expf(m - M);
  const float w2 = m2 == -INFINITY ? 0.f : expf(m2 - M);
  s = s * w1 + s2 * w2;
  m = M;
}

__device__ __forceinline__ RowStat rowstat_merge(RowStat a, const RowStat &b) {
  const bool bw = b.arg.best > a.arg.best || (b.arg.best == a.arg.best && b.arg.idx < a.arg.idx);
  const float zb = bw ? b.zbest : a.zbest;
  a.arg = top2_merge(a.arg, b.arg);
  a.zbest = zb;
  a.zmax = fmaxf(a.zmax, b.zmax);
  ms_merge(a.m, a.s, b.m, b.s);
  return a;
}

__device__ __forceinline__ RowStat rowstat_shfl_xor(const RowStat &a, int o) {
  RowStat b;
  b.arg.best = __shfl_xor(a.arg.best, o, WAVE);
  b.arg.second = __shfl_xor(a.arg.second, o, WAVE);
  b.arg.idx = __shfl_xor(a.arg.idx, o, WAVE);
  b.zbest = __shfl_xor(a.zbest, o, WAVE);
  b.zmax = __shfl_xor(a.zmax, o, WAVE);
  b.m = __shfl_xor(a.m, o, WAVE);
  b.s = __shfl_xor(a.s, o, WAVE);
  return rowstat_merge(a, b);
}

// Reduction of one row's logits held by a lane: NP pairs of 8 consecutive ids
// starting at vw + 32p + 8g.  Writes the logits if asked, draws the Gumbel
// noise (one Philox block per 8 ids; or takes gpre, the same stream's noise
// drawn once for several rows), and returns the lane's statistics merged over
// the wave's four lane groups.
template <int NP, bool STORE = true>
__device__ __forceinline__ RowStat lane_rowstat(const HeadArgs &a, int r, int vw, int g,
                                                float (&zz)[NP][8],
                                                const float (*gpre)[8] = nullptr) {
  const int V = a.vocab;
  const float invT = 1.0f / a.temperature;
  const bool gumbel = a.mode != 0;
  const bool rvalid = r < a.rows;
  const int seq = r / a.rows_per_seq, slot = r % a.rows_per_seq;
  const bool full = vw + 32 * NP <= V;  // wave-uniform: vw is the wave's first id
  RowStat st;
  st.arg.best = -INFINITY;
  st.arg.second = -INFINITY;
  st.arg.idx = 0x7fffffff;
  st.zbest = 0.f;
  st.zmax = -INFINITY;
  st.m = -INFINITY;
  st.s = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int v0 = vw + 32 * p + 8 * g;
    float gn[8];
    if (gpre != nullptr) {
      // noise drawn once for rows that share their stream (shared mode)
#pragma unroll
      for (int e = 0; e < 8; ++e) gn[e] = gpre[p][e];
    } else if (gumbel && rvalid && v0 < V) {
      uint32_t raw[8];
      if (a.mode == 2)
        philox_block8(a.seed, 3u, 0, (uint64_t)slot, a.cycle, (uint64_t)(v0 >> 3), raw);
      else
        philox_block8(a.seed, 0u, (uint64_t)seq, (uint64_t)slot, a.cycle, (uint64_t)(v0 >> 3), raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) gn[e] = gumbel_of(raw[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gn[e] = 0.f;
    }
    // (full: every id of the wave's band lies in the vocabulary, the common
    // case, taken by the whole wave without per-id guards)
    auto push = [&](int e) {
      const int v = v0 + e;
      const float z = zz[p][e];
      const float sc = gumbel ? z * invT + gn[e] : z;
      const bool win = sc > st.arg.best || (sc == st.arg.best && v < st.arg.idx);
      st.zbest = win ? z : st.zbest;
      top2_push(st.arg, sc, v);
      st.zmax = fmaxf(st.zmax, z);
    };
    if (full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) push(e);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (v0 + e < V) push(e);
    }
    if (STORE && a.logits && rvalid) {
      float *lp = a.logits + (long)r * V + v0;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (v0 + e < V) lp[e] = zz[p][e];
    }
  }
  // the largest z / T is the largest z times 1 / T (T > 0; rounding is
  // monotone, so this is exactly the maximum of the rounded products)
  st.m = st.zmax * invT;
  // exp(z / T - m) = exp2(z (log2 e / T) - m log2 e), one FMA per term
  const float kz = invT * 1.4426950408889634f, km = st.m * 1.4426950408889634f;
  if (full && st.m != -INFINITY) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        st.s += __builtin_amdgcn_exp2f(fmaf(zz[p][e], kz, -km));
  } else if (st.m != -INFINITY) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (vw + 32 * p + 8 * g + e < V)
          st.s += __builtin_amdgcn_exp2f(fmaf(zz[p][e], kz, -km));
  }
  st = rowstat_shfl_xor(st, 16);
  st = rowstat_shfl_xor(st, 32);
  return st;
}

__device__ __forceinline__ HeadPartial to_partial(const RowStat &st) {
  HeadPartial hp;
  hp.best = st.arg.best;
  hp.second = st.arg.second;
  hp.idx = st.arg.idx;
  hp.zbest = st.zbest;
  hp.zmax = st.zmax;
  hp.m = st.m;
  hp.s = st.s;
  hp.pad = 0;
  return hp;
}

template <typename T, int MTW>
__global__ __launch_bounds__(256) void lm_head_kernel(HeadArgs a, int nrb) {
  typedef typename Mma<T>::frag F;
  constexpr int VEC = Mma<T>::VEC, KW = Mma<T>::KW;
  __shared__ RowStat red[4][MTW * 16];

  // XCD-aware mapping of the linear workgroup id to (vocab block, row block).
  const int L = blockIdx.x;
  const int xcd = L % NXCD, slot = L / NXCD;
  const int vb = (slot / nrb) * NXCD + xcd, rb = slot % nrb;
  if (vb >= a.nvb) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int vw = vb * HEAD_VB + wave * 64;
  const int rbase = rb * MTW * 16;
  const int V = a.vocab, d = a.d;

  const T *wp[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int v = vw + 32 * (t >> 1) + 8 * (r16 >> 2) + 4 * (t & 1) + (r16 & 3);
    wp[t] = (const T *)a.w + (long)min(v, V - 1) * d + g * VEC;
  }
  const T *xp[MTW];
#pragma unroll
  for (int t = 0; t < MTW; ++t) {
    const int r = min(rbase + 16 * t + r16, a.rows - 1);
    const long hrow = (long)(r / a.rows_per_seq) * a.seq_stride + r % a.rows_per_seq;
    xp[t] = (const T *)a.hidden + hrow * d + g * VEC;
  }

  f32x4 acc[4][MTW];
  stream_mainloop<T, 4, MTW, StreamDepth<4, MTW>::U>(wp, xp, d / KW, acc);

#pragma unroll
  for (int mt = 0; mt < MTW; ++mt) {
    const int r = rbase + 16 * mt + r16;
    float zz[2][8];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) zz[p][e] = acc[2 * p + (e >> 2)][mt][e & 3];
    RowStat st = lane_rowstat<2>(a, r, vw, g, zz);
    if (g == 0) red[wave][16 * mt + r16] = st;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MTW * 16; i += blockDim.x) {
    const int r = rbase + i;
    if (r >= a.rows) continue;
    RowStat st = red[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) st = rowstat_merge(st, red[w][i]);
    a.part[(long)r * a.nvb + vb] = to_partial(st);
  }
}

// LDS-tiled variant (bf16): BN vocabulary ids x BM rows per workgroup on the
// tile engine E.  Up to 160 rows the tile takes every row (each weight tile
// has a single reader) and 64 or 128 ids, which gives many workgroups, so the
// last round of a launch is small next to the others.  At batch scale 256 x 256
// re-uses each staged weight tile across 256 rows.
template <class E>
constexpr int head_stage_wave_rows();

template <class E>
__global__ __launch_bounds__(E::NT) void lm_head_lds_kernel(HeadArgs a, int nmb) {
  constexpr int NW = E::NW, MW = E::MW, BN = E::BN, BM = E::BM;
  __shared__ typename E::Smem sm;
  int vb, rb;
  xcd_block(blockIdx.x, nmb, (a.nvb + 7) >> 3, &vb, &rb);
  if (vb >= a.nvb) return;
  const int v0 = vb * BN, r0 = rb * BM;
  const int V = a.vocab, d = a.d;
  const bf16 *W = (const bf16 *)a.w;
  const bf16 *H = (const bf16 *)a.hidden;
  typename E::Loader ld;
  auto hrow = [&](int r) { return (r / a.rows_per_seq) * a.seq_stride + r % a.rows_per_seq; };
  const int h0 = hrow(r0);
  ld.init(W + (long)v0 * d, [&](int i) { return (min(v0 + i, V - 1) - v0) * d; },
          H + (long)h0 * d, [&](int i) { return (hrow(min(r0 + i, a.rows - 1)) - h0) * d; }, 0);
  f32x4 acc[NW][MW];
  E::template mainloop<true>(sm, ld, d / E::KT, acc);

  // The main loop ended with a barrier: its LDS is free.  The first RED bytes
  // take the per-wave row records; stored logits are staged behind them as
  // [rows][BN + 4] fp32 tiles, WPP wave rows at a time, and written back as
  // whole row runs (a lane's own values are 8 ids of one row, 16 rows per
  // instruction).
  constexpr int LGS = BN + 4;  // staged row stride (floats): 16-row writes hit distinct banks
  constexpr int RED = (E::WN * BM * (int)sizeof(RowStat) + 255) & ~255;  // row-record bytes
  constexpr int WPP = head_stage_wave_rows<E>(), RP = WPP * 16 * MW;
  static_assert(RED + RP * LGS * 4 <= (int)sizeof(typename E::Smem), "logits staging");
  RowStat(*red)[BM] = reinterpret_cast<RowStat(*)[BM]>(&sm);
  float *lg = reinterpret_cast<float *>(reinterpret_cast<char *>(&sm) + RED);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int wn = wave % E::WN, wm = wave / E::WN;
  const int vw = v0 + wn * 16 * NW;
  // lane's values of m-tile mt: 8 consecutive ids vw + 32 p + 8 g .. + 7
  auto lane_vals = [&](int mt, float (&zz)[NW / 2][8]) {
#pragma unroll
    for (int p = 0; p < NW / 2; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) zz[p][e] = acc[2 * p + (e >> 2)][mt][e & 3];
  };
  static_for<MW>([&](auto MT) {
    constexpr int mt = decltype(MT)::value;
    const int rl = wm * 16 * MW + 16 * mt + r16;
    float zz[NW / 2][8];
    lane_vals(mt, zz);
    RowStat st = lane_rowstat<NW / 2, false>(a, r0 + rl, vw, g, zz);
    if (g == 0) red[wn][rl] = st;
  });
  if (a.logits != nullptr) {
#pragma unroll 1
    for (int p = 0; p < E::WM / WPP; ++p) {
      if (wm / WPP == p) {
        static_for<MW>([&](auto MT) {
          constexpr int mt = decltype(MT)::value;
          float zz[NW / 2][8];
          lane_vals(mt, zz);
          const int rs = (wm % WPP) * 16 * MW + 16 * mt + r16;
#pragma unroll
          for (int q = 0; q < NW / 2; ++q) {
            float *dst = lg + rs * LGS + wn * 16 * NW + 32 * q + 8 * g;
            *reinterpret_cast<f32x4 *>(dst) = f32x4{zz[q][0], zz[q][1], zz[q][2], zz[q][3]};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{zz[q][4], zz[q][5], zz[q][6], zz[q][7]};
          }
        });
      }
      __syncthreads();
      for (int i = threadIdx.x; i < RP * (BN / 4); i += E::NT) {
        const int rl = i / (BN / 4), v = v0 + 4 * (i % (BN / 4)), r = r0 + p * RP + rl;
        if (r >= a.rows || v >= V) continue;
        const f32x4 x = *reinterpret_cast<const f32x4 *>(lg + rl * LGS + (v - v0));
        float *dst = a.logits + (long)r * V + v;
        if (v + 4 <= V && (V & 3) == 0) {
          // streaming store: the logits are read back at most one row per
          // sequence, long after, so they should not displace weight tiles
          // that the other row blocks still read through L2
          __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(dst));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < V) dst[e] = x[e];
        }
      }
      if (p + 1 < E::WM / WPP) __syncthreads();
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < BM; i += E::NT) {
    const int r = r0 + i;
    if (r >= a.rows) continue;
    RowStat st = red[0][i];
#pragma unroll
    for (int w = 1; w < E::WN; ++w) st = rowstat_merge(st, red[w][i]);
    a.part[(long)r * a.nvb + vb] = to_partial(st);
  }
}

// Wave rows staged per pass of the logits store: the most that fit behind
// the row records.
template <class E>
constexpr int head_stage_wave_rows() {
  const long red = ((long)E::WN * E::BM * sizeof(RowStat) + 255) & ~255L;
  int w = E::WM;
  while (w > 1 && (E::WM % w != 0 ||
                   red + (long)w * 16 * E::MW * (E::BN + 4) * 4 > (long)sizeof(typename E::Smem)))
    --w;
  return w;
}

// Weight-streaming variant for up to 160 rows (bf16): the weight tile of 128
// vocabulary rows streams through a ring of LDS stages (the 2 KS contiguous
// bytes of every row), filled by direct global->LDS copies NS - 1 stages
// ahead; the slice of the 16 RT hidden rows rides in the same ring.  Up to
// 64 rows the stages are 128 deep (four stages up to 32 rows, three beyond);
// from 65 rows 64 deep, four stages (measured on the 8B-shaped head at 144
// rows: 397 us for the 128 x 160 tile of the tile engine, 371 us here in
// argmax mode; two vocabulary tile pairs per wave, 256 ids per workgroup,
// took 403 us: 594 workgroups round to three passes over 256 compute units).
// The kernel also takes several row blocks, those of one vocabulary block
// placed on one XCD next to each other (workgroup i runs on XCD i mod 8); the
// launch uses one.  LDS rows are unpadded and XOR-swizzled per 16-byte chunk,
// so the 16 rows one fragment read touches (in the permuted vocabulary order)
// fall on distinct banks.
constexpr int HS_MAX_RT = 10;   // row tiles of 16 per workgroup

// Stage geometry: TPW pairs of 16-id vocabulary tiles per wave (HS rows =
// 128 TPW per workgroup of 4 waves), KS = k per stage: 128 with one pair (up
// to 4 row tiles), 64 with two pairs (5 to 10 row tiles: each hidden
// fragment read from LDS feeds four products instead of two, and the 80-160
// hidden rows of a stage still leave room for a three-deep ring).  A stage
// row is 2 KS bytes; one copy (64 lanes x 16 bytes) fills 512 / KS rows.
template <int RT, int KS, int TPW>
struct HsStage {
  bf16 w[128 * TPW * KS];
  bf16 x[16 * RT * KS];
};
template <int RT, int KS, int TPW>
constexpr int hs_stages() {
  constexpr int n = (int)((160 * 1024) / sizeof(HsStage<RT, KS, TPW>));
  return n < 4 ? n : 4;
}
static_assert(hs_stages<2, 128, 1>() == 4 && hs_stages<4, 128, 1>() == 3, "ring depths");
static_assert(hs_stages<10, 64, 1>() == 4, "ring depth of the 160-row slices");

// 16-byte chunk swizzles.  KS = 128 (16 chunks per row): weight rows on
// bits {0, 1, 3, 4}, the bits that vary over the 16 (permuted) rows of one
// fragment read; hidden rows on bits 0..3.  KS = 64 (8 chunks, two rows per
// 256-byte bank window): weight rows on bits {1, 3, 4}, hidden rows on bits
// {1, 2, 3} (bit 0 picks the half of the bank window).
template <int KS>
__device__ __forceinline__ int hs_wswz(int row) {
  if (KS == 128) return (row & 3) | ((row >> 1) & 12);
  return ((row >> 1) & 1) | ((row >> 2) & 6);
}
template <int KS>
__device__ __forceinline__ int hs_xswz(int row) {
  if (KS == 128) return row & 15;
  return (row >> 1) & 7;
}

template <int RT, int KS, int TPW>
__global__ __launch_bounds__(256) void lm_head_stream_kernel(HeadArgs a, int nrb) {
  constexpr int ROWS = 128 * TPW;                               // vocabulary rows per workgroup
  constexpr int CPR = KS / 8, CROWS = 64 / CPR;                 // chunks per row, rows per copy
  constexpr int WC = ROWS * KS * 2 / 1024 / 4;                  // weight copies per wave per stage
  constexpr int XC = 16 * RT * KS * 2 / 1024 / 4;               // hidden copies per wave per stage
  static_assert(16 * RT * KS * 2 % 4096 == 0, "hidden copies split evenly over the 4 waves");
  constexpr int NS = hs_stages<RT, KS, TPW>(), OPS = WC + XC;   // copies per wave per stage
  static_assert(NS >= 2, "ring");
  __shared__ HsStage<RT, KS, TPW> ring[NS];
  // XCD-aware mapping of the linear workgroup id to (vocab block, row block)
  const int L = blockIdx.x;
  const int xcd = L % NXCD, slot = L / NXCD;
  const int vb = (slot / nrb) * NXCD + xcd, rb = slot % nrb;
  if (vb >= a.nvb) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int V = a.vocab, d = a.d;
  const int v0 = vb * ROWS, r0 = rb * 16 * RT;
  auto hrow = [&](int r) { return (long)(r / a.rows_per_seq) * a.seq_stride + r % a.rows_per_seq; };
  const long h0 = hrow(r0);
  const char *wblk = reinterpret_cast<const char *>((const bf16 *)a.w + (long)v0 * d);
  const char *xblk = reinterpret_cast<const char *>((const bf16 *)a.hidden + h0 * d);
  // copy j of wave w fills LDS vectors 64 (4 j + w) + lane: stage row
  // CROWS (4 j + w) + lane / CPR, physical chunk lane % CPR (weight and
  // hidden alike, each in its own part of the stage)
  uint32_t goff[WC];
#pragma unroll
  for (int j = 0; j < WC; ++j) {
    const int row = CROWS * (4 * j + wave) + lane / CPR, pc = lane % CPR;
    goff[j] = (uint32_t)((min(v0 + row, V - 1) - v0) * d * 2 + 16 * (pc ^ hs_wswz<KS>(row)));
  }
  uint32_t xoff[XC];
#pragma unroll
  for (int j = 0; j < XC; ++j) {
    const int row = CROWS * (4 * j + wave) + lane / CPR, pc = lane % CPR;
    const int r = min(r0 + row, a.rows - 1);
    xoff[j] = (uint32_t)((hrow(r) - h0) * d * 2 + 16 * (pc ^ hs_xswz<KS>(row)));
  }
  // A-operand rows of this wave's tiles (permuted vocabulary order: tile
  // 2q + t row 4 i + e is id 32 q + 8 i + 4 t + e of the wave's band)
  int arow[2 * TPW];
#pragma unroll
  for (int t = 0; t < 2 * TPW; ++t)
    arow[t] = 32 * (TPW * wave + (t >> 1)) + 8 * (r16 >> 2) + 4 * (t & 1) + (r16 & 3);
  f32x4 acc[2 * TPW][RT];
#pragma unroll
  for (int t = 0; t < 2 * TPW; ++t)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = d / KS;
  // each block starts its k walk at a different stage, so concurrent blocks
  // do not sweep the same column offset of their rows at the same time (the
  // row blocks of one vocabulary block share the start, so they read the
  // same weight bytes at about the same time)
  const int rot = (vb * 5) % nst;
  auto kst = [&](int s) { return s + rot < nst ? s + rot : s + rot - nst; };
  auto issue = [&](int s) {
    const long k0 = (long)kst(s) * KS * 2;
    HsStage<RT, KS, TPW> &st = ring[s % NS];
    const uint32_t wl = lds_u32(&st.w[0]) + wave * 1024;
#pragma unroll
    for (int j = 0; j < WC; ++j) dma16(wblk + k0, goff[j], wl + j * 4096);
    const uint32_t xl = lds_u32(&st.x[0]) + wave * 1024;
#pragma unroll
    for (int j = 0; j < XC; ++j) dma16(xblk + k0, xoff[j], xl + j * 4096);
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nst) issue(p);
  for (int s = 0; s < nst; ++s) {
    // stage s has landed once at most the copies of the stages after it (up
    // to NS - 2 of them) are outstanding
    const int ahead = min(nst - 1 - s, NS - 2);
    if (ahead >= 2) wait_vmcnt<2 * OPS>();
    else if (ahead == 1) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    // every wave's copies of stage s are visible, and the buffer refilled
    // next (read at stage s - 1) is free
    __syncthreads();
    if (s + NS - 1 < nst) issue(s + NS - 1);
    // (written out here rather than in a lambda over acc: with many row
    // tiles the compiler would keep a captured accumulator array in memory)
    const char *ws = reinterpret_cast<const char *>(&ring[s % NS].w[0]);
    const char *xs = reinterpret_cast<const char *>(&ring[s % NS].x[0]);
#pragma unroll
    for (int kk = 0; kk < KS / 32; ++kk) {
      bf16x8 xf[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        xf[rt] = *reinterpret_cast<const bf16x8 *>(
            xs + (16 * rt + r16) * KS * 2 + 16 * ((kk * 4 + g) ^ hs_xswz<KS>(16 * rt + r16)));
#pragma unroll
      for (int t = 0; t < 2 * TPW; ++t) {
        const bf16x8 fa = *reinterpret_cast<const bf16x8 *>(
            ws + arow[t] * KS * 2 + 16 * ((kk * 4 + g) ^ hs_wswz<KS>(arow[t])));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[t][rt] = Mma<bf16>::run(fa, xf[rt], acc[t][rt]);
      }
    }
  }
  __syncthreads();
  // epilogue: per row, the wave's 32 TPW ids, then the four waves in LDS
  RowStat(*red)[16 * RT] = reinterpret_cast<RowStat(*)[16 * RT]>(&ring[0]);
  static_assert(4 * 16 * RT * sizeof(RowStat) <= sizeof(ring), "row records fit the ring");
  const int vw = v0 + 32 * TPW * wave;
  // Shared-noise mode draws one stream per block slot: when the slots of
  // this lane's rows 16 rt + r16 are all r16 % rows_per_seq (rows_per_seq
  // divides 16), the lane draws that stream's noise once for all its rows.
  float gsh[TPW][8];
  const bool share = a.mode == 2 && 16 % a.rows_per_seq == 0;
  if (share) {
    const int sl = r16 % a.rows_per_seq;
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const int gv0 = vw + 32 * p + 8 * g;
      uint32_t raw[8];
      philox_block8(a.seed, 3u, 0, (uint64_t)sl, a.cycle, (uint64_t)(gv0 >> 3), raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) gsh[p][e] = gv0 < V ? gumbel_of(raw[e]) : 0.f;
    }
  }
  // (a compile-time loop: a rolled one would index acc at run time and put
  // it in memory)
  static_for<RT>([&](auto RTI) {
    constexpr int rt = decltype(RTI)::value;
    float zz[TPW][8];
#pragma unroll
    for (int p = 0; p < TPW; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) zz[p][e] = acc[2 * p + (e >> 2)][rt][e & 3];
    RowStat st2 = lane_rowstat<TPW>(a, r0 + 16 * rt + r16, vw, g, zz, share ? gsh : nullptr);
    if (g == 0) red[wave][16 * rt + r16] = st2;
  });
  __syncthreads();
  if (threadIdx.x < 16 * RT && r0 + (int)threadIdx.x < a.rows) {
    const int i = threadIdx.x;
    RowStat t = red[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) t = rowstat_merge(t, red[w][i]);
    a.part[(long)(r0 + i) * a.nvb + vb] = to_partial(t);
  }
}

template <int RT, int KS, int TPW>
static void launch_stream(const HeadArgs &a, int nrb, hipStream_t st) {
  const dim3 grid((a.nvb + NXCD - 1) / NXCD * NXCD * nrb);
  hipLaunchKernelGGL((lm_head_stream_kernel<RT, KS, TPW>), grid, dim3(256), 0, st, a, nrb);
}

// One workgroup per row merges the row's vocabulary-block records in two
// passes over them: the top-2 / zmax / largest block maximum M, then the
// fp64 sum of s_i exp(m_i - M) (one exponential per record, no dependent
// chain).  Each thread takes records tid, tid + COMB_T, ... in order, then
// the waves reduce by a fixed butterfly and the four wave results merge in
// wave order: deterministic.
constexpr int COMB_T = 256;

__device__ __forceinline__ void arg_merge(ArgTop2 &arg, float &zbest, const ArgTop2 &o, float zb) {
  const bool bw = o.best > arg.best || (o.best == arg.best && o.idx < arg.idx);
  if (bw) zbest = zb;
  arg = top2_merge(arg, o);
}

__global__ __launch_bounds__(COMB_T) void lm_combine_kernel(HeadArgs a) {
  constexpr int NWV = COMB_T / 64;
  __shared__ ArgTop2 s_arg[NWV];
  __shared__ float s_zb[NWV], s_zmax[NWV], s_m[NWV];
  __shared__ double s_s[NWV];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const HeadPartial *p = a.part + (long)r * a.nvb;
  ArgTop2 arg;
  arg.best = -INFINITY;
  arg.second = -INFINITY;
  arg.idx = 0x7fffffff;
  float zbest = 0.f, zmax = -INFINITY, m = -INFINITY;
  // records in batches of CB per thread, loaded before any is merged; the
  // (m, s) of the first batch stay in registers for the second pass, which
  // then needs no reload when one batch covers the row (nvb <= CB COMB_T)
  constexpr int CB = 8;
  float bm[CB], bs[CB];
  for (int i0 = 0; i0 < a.nvb; i0 += CB * COMB_T) {
    HeadPartial hb[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int i = i0 + tid + u * COMB_T;
      if (i < a.nvb) hb[u] = p[i];
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int i = i0 + tid + u * COMB_T;
      if (i0 == 0) {
        bm[u] = i < a.nvb ? hb[u].m : -INFINITY;
        bs[u] = i < a.nvb ? hb[u].s : 0.f;
      }
      if (i >= a.nvb) continue;
      ArgTop2 o;
      o.best = hb[u].best;
      o.second = hb[u].second;
      o.idx = hb[u].idx;
      arg_merge(arg, zbest, o, hb[u].zbest);
      zmax = fmaxf(zmax, hb[u].zmax);
      m = fmaxf(m, hb[u].m);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    ArgTop2 b;
    b.best = __shfl_xor(arg.best, o, WAVE);
    b.second = __shfl_xor(arg.second, o, WAVE);
    b.idx = __shfl_xor(arg.idx, o, WAVE);
    arg_merge(arg, zbest, b, __shfl_xor(zbest, o, WAVE));
    zmax = fmaxf(zmax, __shfl_xor(zmax, o, WAVE));
    m = fmaxf(m, __shfl_xor(m, o, WAVE));
  }
  if (lane == 0) {
    s_arg[wave] = arg;
    s_zb[wave] = zbest;
    s_zmax[wave] = zmax;
    s_m[wave] = m;
  }
  __syncthreads();
  float M = s_m[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) M = fmaxf(M, s_m[w]);
  double s = 0.0;
  if (M != -INFINITY) {
    // same order as before: record tid, tid + COMB_T, ...
#pragma unroll
    for (int u = 0; u < CB; ++u)
      if (bm[u] != -INFINITY) s += (double)bs[u] * exp((double)bm[u] - (double)M);
    for (int i = tid + CB * COMB_T; i < a.nvb; i += COMB_T) {
      const float mi = p[i].m, si = p[i].s;
      if (mi != -INFINITY) s += (double)si * exp((double)mi - (double)M);
    }
  }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, WAVE);
  if (lane == 0) s_s[wave] = s;
  __syncthreads();
  if (tid == 0) {
    ArgTop2 g = s_arg[0];
    float zb = s_zb[0], zm = s_zmax[0];
    double S = s_s[0];
    for (int w = 1; w < NWV; ++w) {
      arg_merge(g, zb, s_arg[w], s_zb[w]);
      zm = fmaxf(zm, s_zmax[w]);
      S += s_s[w];
    }
    a.ids[r] = g.idx;
    if (a.zmax) a.zmax[r] = zm;
    if (a.lse) a.lse[r] = (float)((double)M + log(S));
    if (a.zsel) a.zsel[r] = zb;
    if (a.gap) a.gap[r] = g.best - g.second;
  }
}

template <typename T, int MTW>
static void launch_typed(const HeadArgs &a, hipStream_t st) {
  const int nrb = (a.rows + MTW * 16 - 1) / (MTW * 16);
  const int nvb8 = (a.nvb + NXCD - 1) / NXCD * NXCD;
  hipLaunchKernelGGL((lm_head_kernel<T, MTW>), dim3(nvb8 * nrb), dim3(256), 0, st, a, nrb);
}

template <typename T>
static void launch_rows(const HeadArgs &a, hipStream_t st) {
  if (a.rows <= 16) launch_typed<T, 1>(a, st);
  else if (a.rows <= 32) launch_typed<T, 2>(a, st);
  else if (a.rows <= 48) launch_typed<T, 3>(a, st);
  else launch_typed<T, 4>(a, st);
}

template <class E>
static void launch_head_tile(const HeadArgs &a, dim3 grid, int nmb, hipStream_t st) {
  hipLaunchKernelGGL((lm_head_lds_kernel<E>), grid, dim3(E::NT), 0, st, a, nmb);
}

void launch_lm_head(const HeadArgs &args, hipStream_t st) {
  if (args.rows == 0) return;
  HeadArgs a = args;
  // up to 160 rows stream the weight through an LDS ring; more rows (and,
  // up to 64 rows, depths the 128-deep streaming stages do not divide) go
  // through the tile engine, with a tile fitted to the row count (both
  // address a block's hidden rows with 32-bit byte offsets).  From 65 to 160
  // rows the streaming conditions hold whenever the tile's do (64-deep
  // stages, a span no larger than the tile's), so no tile serves them.
  int BN = HeadBigTile::BN, BM = HeadBigTile::BM;
  if (a.rows <= 32) BN = 64, BM = 32;
  else if (a.rows <= 64) BN = 64, BM = 64;
  const long span = ((long)(BM - 1) / a.rows_per_seq + 1) * a.seq_stride * a.d * 2;
  // streaming path: up to 160 rows, one row block of 16 RT rows (measured on
  // the 8B-shaped head: 30 rows 306 -> 248 us, 60 rows 298 -> 273 us against
  // the 64 x 32 / 64 x 64 tiles; 144 rows 397 -> 371 us against 128 x 160)
  const int snrb = 1, srt = (a.rows + 15) / 16;
  const long sspan = ((long)(16 * srt - 1) / a.rows_per_seq + 1) * a.seq_stride * a.d * 2;
  const int sks = srt <= 4 ? 128 : 64;
  if (a.dtype == 1 && a.rows <= 16 * HS_MAX_RT && a.d % sks == 0 && sspan < (1L << 31)) {
    a.nvb = (a.vocab + 127) / 128;
    if (srt == 1) launch_stream<1, 128, 1>(a, snrb, st);
    else if (srt == 2) launch_stream<2, 128, 1>(a, snrb, st);
    else if (srt == 3) launch_stream<3, 128, 1>(a, snrb, st);
    else if (srt == 4) launch_stream<4, 128, 1>(a, snrb, st);
    else if (srt <= 6) launch_stream<6, 64, 1>(a, snrb, st);
    else if (srt <= 8) launch_stream<8, 64, 1>(a, snrb, st);
    else launch_stream<10, 64, 1>(a, snrb, st);
  } else if (a.dtype == 1 && a.d % HEAD_KT == 0 && span < (1L << 31)) {
    a.nvb = (a.vocab + BN - 1) / BN;
    const int nmb = (a.rows + BM - 1) / BM;
    const dim3 grid((a.nvb + NXCD - 1) / NXCD * NXCD * nmb);
    if (BM == 32) launch_head_tile<HeadTile<2, 1>>(a, grid, nmb, st);
    else if (BM == 64) launch_head_tile<HeadTile<2, 2>>(a, grid, nmb, st);
    else launch_head_tile<HeadBigTile>(a, grid, nmb, st);
  } else {
    a.nvb = (a.vocab + HEAD_VB - 1) / HEAD_VB;
    if (a.dtype == 1) launch_rows<bf16>(a, st);
    else launch_rows<float>(a, st);
  }
  hipLaunchKernelGGL(lm_combine_kernel, dim3(a.rows), dim3(COMB_T), 0, st, a);
}

}  // namespace dstill
