// Non-causal block attention over the injected context (DFlash review,
// Method / Inference: K_i = [W^K H_t ; W^K H_d], V_i likewise, the block
// attending bidirectionally; DStill, Setup and notation: context strictly
// before the anchor).  Each query of copy c of sequence b attends
//   [cached K/V rows 0 .. S_b-1 ; the B block keys of copy c]
// with no mask (SPOT, Method: a copy sees the prefix and itself only),
// scaled by 1/sqrt(dh), through a softmax over all S_b + B keys.
//
// Work decomposition ("split context"): one workgroup per (split, kv head,
// sequence-copy), placed by split_coords.  Its query waves each own one
// query head of the GQA group, i.e. B <= 16 query rows (one 16-row MFMA
// tile).  The workgroup walks its context range in chunks of 64 keys,
// computes S^T = K Q^T and O^T = V^T P^T on the matrix cores and keeps an
// online softmax per query; split 0 also takes the block keys.  The V cache
// is stored in tiles of 64 keys, each d-major ([cap/64][dh][64] per sequence
// and head), so V^T of a chunk is one contiguous 16 KB block, like the chunk
// of K.  bf16 chunks stream through a ring of LDS buffers filled by direct
// global->LDS copies (attn_split_dma_kernel); fp32 chunks, and bf16 shapes
// whose copies do not split evenly over the waves, are staged through
// registers (attn_split_kernel).  The partial (m, l, O) of every split is
// merged by attn_combine with the log-sum-exp rule, which reproduces the
// single softmax up to rounding.
//
// Lane layout (see Mma in common.hpp): in S^T, lane l holds query l % 16 and,
// with the key rows of each 32-key sub-chunk permuted so that tile t row
// 4g + i is key 8g + 4t + i, the 8 consecutive keys 8g .. 8g+7 (g = l / 16).
// Those 8 probabilities are exactly that lane's B fragment of P^T, and the
// matching A fragment of V^T is 8 consecutive keys of one V^T row.  The row
// max/sum over a query's keys is then a reduction over the four lane
// groups: two xor-shuffles (16, 32).
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "kernels.hpp"

namespace dstill {

constexpr int ATT_KC = 64;  // keys per LDS chunk
constexpr int ATT_VBS = 16;  // key stride of the block V^T workspace

// Two LDS buffers of one chunk: K row-major [key][dh], V^T [dh][key]; rows
// padded by 16 bytes so fragment reads of 16 rows hit distinct banks.
template <typename T, int DH>
struct AttnSmem {
  static constexpr int VEC = Mma<T>::VEC;
  static constexpr int KS = DH + VEC;
  static constexpr int VS = ATT_KC + VEC;
  T k[2][ATT_KC * KS];
  T vt[2][DH * VS];
};

// Copies one chunk global -> registers (issued early) -> LDS (after the
// current chunk's compute).  K rows are contiguous dh-vectors; a V tile is
// d-major, so a V^T row of the chunk is 64 consecutive keys of one d.  Loads
// are unconditional from clamped, in-bounds addresses (no branch, so nothing
// waits on them until the store); keys at or beyond nk are masked at store
// time: V to zero so no stale value reaches P.V, K left as is (its scores are
// replaced by -inf).
template <typename T, int DH, int NTHR>
struct ChunkLoader {
  typedef typename Mma<T>::frag F;
  static constexpr int VEC = Mma<T>::VEC;
  static constexpr int NV = ATT_KC * DH / VEC / NTHR;  // vectors of K (and of V) per thread
  F kr[NV], vr[NV];
  int nk;

  __device__ __forceinline__ void load(const T *__restrict__ ksrc, long kstride,
                                       const T *__restrict__ vsrc, long vstride, int nkeys) {
    nk = nkeys;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int item = threadIdx.x + NTHR * i;
      const int key = min(item / (DH / VEC), nk - 1), c = (item % (DH / VEC)) * VEC;
      kr[i] = load_frag<T>(ksrc + key * kstride + c);
      const int d = item / (ATT_KC / VEC), kc = (item % (ATT_KC / VEC)) * VEC;
      // a vector starting below nk stays inside the row (rows hold a multiple of 8)
      vr[i] = load_frag<T>(vsrc + d * vstride + (kc < nk ? kc : 0));
    }
  }
  __device__ __forceinline__ void store(AttnSmem<T, DH> &sm, int buf) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int item = threadIdx.x + NTHR * i;
      const int key = item / (DH / VEC), c = (item % (DH / VEC)) * VEC;
      *reinterpret_cast<F *>(&sm.k[buf][key * AttnSmem<T, DH>::KS + c]) = kr[i];
      const int d = item / (ATT_KC / VEC), kc = (item % (ATT_KC / VEC)) * VEC;
      if (nk < ATT_KC) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (kc + e >= nk) vr[i][e] = T(0.0f);
      }
      *reinterpret_cast<F *>(&sm.vt[buf][d * AttnSmem<T, DH>::VS + kc]) = vr[i];
    }
  }
};

// Where a chunk's elements sit in LDS.  PadLayout: the register-staged
// buffers above (rows padded by one vector).  SwzLayout (bf16): the ring
// buffers filled by direct copies, unpadded, 16-byte chunk c of a row at
// chunk c ^ swz(row): K rows (dh * 2 bytes) swizzled on key bits
// {0, 1, 3, 4}, the bits that vary across the 16 keys one fragment read
// touches (see attend_chunk); V^T rows (128 bytes, two per 256-byte bank
// window) on bits {1, 2, 3} of d.
template <typename T, int DH>
struct PadLayout {
  static __device__ __forceinline__ const T *k(const T *base, int key, int col) {
    return base + key * AttnSmem<T, DH>::KS + col;
  }
  static __device__ __forceinline__ const T *v(const T *base, int d, int key) {
    return base + d * AttnSmem<T, DH>::VS + key;
  }
};

template <int DH>
struct SwzLayout {
  static __device__ __forceinline__ int kswz(int key) {
    if (DH == 128) return (key & 3) | (((key >> 3) & 3) << 2);
    return ((key >> 1) & 1) | (((key >> 3) & 3) << 1);
  }
  static __device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }
  static __device__ __forceinline__ int kbyte(int key, int chunk) {
    return key * DH * 2 + ((chunk ^ kswz(key)) << 4);
  }
  static __device__ __forceinline__ int vbyte(int d, int chunk) {
    return d * ATT_KC * 2 + ((chunk ^ vswz(d)) << 4);
  }
  static __device__ __forceinline__ const bf16 *k(const bf16 *base, int key, int col) {
    return reinterpret_cast<const bf16 *>(reinterpret_cast<const char *>(base) +
                                          kbyte(key, col >> 3));
  }
  static __device__ __forceinline__ const bf16 *v(const bf16 *base, int d, int key) {
    return reinterpret_cast<const bf16 *>(reinterpret_cast<const char *>(base) +
                                          vbyte(d, key >> 3));
  }
};

template <typename T, int DH>
struct WaveState {
  float m, l;
  f32x4 o[DH / 16];
};

// Online-softmax reference update for a new block of scores with per-query
// max cmax (finite).  The reference m moves only when some query's max
// exceeds it by more than RESCALE_LOG2 in log2 units (a wave-uniform branch);
// until then probabilities up to 2^RESCALE_LOG2 accumulate against the old
// reference, which l and O share, so their ratio is unchanged.  A split
// starts at m = -inf and takes the first block's max.
constexpr float RESCALE_LOG2 = 8.0f;

template <int DH, typename WS>
__device__ __forceinline__ void rescale(WS &ws, float cmax, float c) {
  if (__any((cmax - ws.m) * c > RESCALE_LOG2)) {
    const float mnew = fmaxf(ws.m, cmax);
    const float alpha = __builtin_amdgcn_exp2f((ws.m - mnew) * c);
    ws.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) ws.o[dt] *= alpha;
    ws.m = mnew;
  }
}

// Workgroup -> (split, kv head, sequence-copy).  Items are numbered with the
// split index slowest, item = sp * pairs + bc * hkv + h; the workgroups take
// them in the order of a work list sorted by decreasing chunk count (built
// once per call by attn_worklist_kernel), so full splits start first and the
// short last splits of each context fill the tail.  Consecutive workgroups go
// round-robin to the 8 XCDs, so each XCD gets an even share of the work.
__device__ __forceinline__ void split_coords(const AttnArgs &a, int *sp, int *h, int *bc) {
  const int pairs = a.hkv * a.bs * a.C;
  const int L = a.worklist ? a.worklist[blockIdx.x] : (int)blockIdx.x;
  *sp = L / pairs;
  *h = (L % pairs) % a.hkv;
  *bc = (L % pairs) / a.hkv;
}

// Context range of a sequence under the sliding window: the first visible
// key, and the chunk-aligned start the splits count from (the V cache is
// tiled in 64-key tiles); keys between the two are masked in the first chunk.
__device__ __forceinline__ int ctx_first(int S, int window) {
  return window > 0 && S > window ? S - window : 0;
}
__device__ __forceinline__ int ctx_lo(int S, int window) {
  return ctx_first(S, window) & ~(ATT_KC - 1);
}

// Counting sort of the items by decreasing number of 64-key context chunks
// (split 0 counts one more for the block keys; empty splits go last).  One
// workgroup; the order within a count is whatever the atomics give, which
// changes nothing but the schedule.
__global__ __launch_bounds__(1024) void attn_worklist_kernel(AttnArgs a, int *__restrict__ list) {
  constexpr int NB = 130;  // counts 0 .. 129 (split <= 128 chunks, + the block chunk)
  __shared__ int hist[NB], base[NB];
  const int pairs = a.hkv * a.bs * a.C, n = a.nsplit * pairs;
  for (int i = threadIdx.x; i < NB; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  auto count = [&](int L) {
    const int sp = L / pairs, bc = (L % pairs) / a.hkv;
    const int S = a.eff_ctx[bc / a.C];
    const int k0 = ctx_lo(S, a.window) + sp * a.split, k1 = min(k0 + a.split, S);
    const int c = k1 > k0 ? (k1 - k0 + ATT_KC - 1) / ATT_KC : 0;
    return min(c + (sp == 0 ? 1 : 0), NB - 1);
  };
  for (int L = threadIdx.x; L < n; L += blockDim.x) atomicAdd(&hist[count(L)], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int c = NB - 1; c >= 0; --c) {
      base[c] = acc;
      acc += hist[c];
    }
  }
  __syncthreads();
  for (int L = threadIdx.x; L < n; L += blockDim.x) list[atomicAdd(&base[count(L)], 1)] = L;
}

// One wave's pass over a staged chunk holding valid keys kf..nk-1 (nk in
// 1..64; kf > 0 only in the first chunk under a sliding window, with at least
// one valid key), with one online-softmax update for the whole chunk.  Scores stay in raw units
// (m is the reference max of raw scores); probabilities are
// exp2(s * c - m * c) with c = log2(e) / sqrt(dh), one FMA and one v_exp_f32
// each.
template <typename T, int DH, class Lay>
__device__ __forceinline__ void attend_chunk(const T *__restrict__ ks_lds,
                                             const T *__restrict__ vt_lds,
                                             const typename Mma<T>::frag *qf, int nk, int kf,
                                             float c, WaveState<T, DH> &ws) {
  constexpr int VEC = Mma<T>::VEC, KW = Mma<T>::KW;
  typedef typename Mma<T>::frag F;
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int nsub = nk > 32 ? 2 : 1;  // 32-key sub-chunks holding a valid key
  // S^T tiles: tile t covers sub-chunk t >> 1; lane holds keys
  // 32 (t >> 1) + 8 g + 4 (t & 1) + i, i = 0..3
  f32x4 s[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s[t] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if ((t >> 1) < nsub) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int krow = 32 * (t >> 1) + 8 * (r16 >> 2) + 4 * (t & 1) + (r16 & 3);
#pragma unroll
      for (int ks = 0; ks < DH / KW; ++ks)
        s[t] = Mma<T>::run(*reinterpret_cast<const F *>(Lay::k(ks_lds, krow, ks * KW + VEC * g)),
                           qf[ks], s[t]);
    }
  }
  if (nk < ATT_KC || kf > 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i;
        if (key >= nk || key < kf) s[t][i] = -INFINITY;
      }
  }
  float cmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  cmax = fmaxf(cmax, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                           fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, WAVE));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, WAVE));
  rescale<DH>(ws, cmax, c);
  const float mc = ws.m * c;
  float p[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[t][i] = __builtin_amdgcn_exp2f(fmaf(s[t][i], c, -mc));
      ws.l += p[t][i];
    }
  // P^T fragments per sub-chunk: keys 8g .. 8g+7 are p[2sc][0..3], p[2sc+1][0..3].
  // bf16 carries each probability as three terms hi + mid + lo (each the
  // bf16 rounding of what the previous ones leave), so P.V sees the full fp32
  // probability (8 + 8 + 8 significant bits); fp32 uses two exact fragments.
  constexpr int NPF = 8 / VEC;
  constexpr bool SPLIT = VEC == 8;
#pragma unroll
  for (int sc = 0; sc < 2; ++sc) {
    if (sc >= nsub) break;
    F pf[NPF], pm[NPF], pl[NPF];
#pragma unroll
    for (int f = 0; f < NPF; ++f)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int k8 = f * VEC + e;  // 0..7
        const float pv = p[2 * sc + (k8 >> 2)][k8 & 3];
        const T hi = from_f32<T>(pv);
        pf[f][e] = hi;
        if (SPLIT) {
          const float r1 = pv - to_f32(hi);
          const T mid = from_f32<T>(r1);
          pm[f][e] = mid;
          pl[f][e] = from_f32<T>(r1 - to_f32(mid));
        }
      }
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
#pragma unroll
      for (int f = 0; f < NPF; ++f) {
        const F vf =
            *reinterpret_cast<const F *>(Lay::v(vt_lds, dt * 16 + r16, sc * 32 + 8 * g + f * VEC));
        if (SPLIT) {
          ws.o[dt] = Mma<T>::run(vf, pl[f], ws.o[dt]);
          ws.o[dt] = Mma<T>::run(vf, pm[f], ws.o[dt]);
        }
        ws.o[dt] = Mma<T>::run(vf, pf[f], ws.o[dt]);
      }
    }
  }
}

// One wave's pass over the 32-key sub-chunk `sub` of a staged chunk, of which
// keys kf..nk-1 (nk in 1..32; kf > 0 only under a sliding window) are valid: two S^T tiles, one online-softmax
// update, one P.V pass (same lane layout as attend_chunk).
template <int DH, class Lay>
__device__ __forceinline__ void attend_sub(const bf16 *__restrict__ ks_lds,
                                           const bf16 *__restrict__ vt_lds, const bf16x8 *qf,
                                           int sub, int nk, int kf, float c,
                                           WaveState<bf16, DH> &ws) {
  typedef bf16x8 F;
  constexpr int KW = 32;
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  f32x4 s[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int krow = 32 * sub + 8 * (r16 >> 2) + 4 * t + (r16 & 3);
#pragma unroll
    for (int ks = 0; ks < DH / KW; ++ks)
      s[t] = Mma<bf16>::run(*reinterpret_cast<const F *>(Lay::k(ks_lds, krow, ks * KW + 8 * g)),
                            qf[ks], s[t]);
  }
  if (nk < 32 || kf > 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 8 * g + 4 * t + i;
        if (key >= nk || key < kf) s[t][i] = -INFINITY;
      }
  }
  float cmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, WAVE));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, WAVE));
  rescale<DH>(ws, cmax, c);
  const float mc = ws.m * c;
  F pf, pm, pl;
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) {
    const float pv = __builtin_amdgcn_exp2f(fmaf(s[k8 >> 2][k8 & 3], c, -mc));
    ws.l += pv;
    const bf16 hi = from_f32<bf16>(pv);
    const float r1 = pv - to_f32(hi);
    const bf16 mid = from_f32<bf16>(r1);
    pf[k8] = hi;
    pm[k8] = mid;
    pl[k8] = from_f32<bf16>(r1 - to_f32(mid));
  }
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) {
    const F vf = *reinterpret_cast<const F *>(Lay::v(vt_lds, dt * 16 + r16, sub * 32 + 8 * g));
    ws.o[dt] = Mma<bf16>::run(vf, pl, ws.o[dt]);
    ws.o[dt] = Mma<bf16>::run(vf, pm, ws.o[dt]);
    ws.o[dt] = Mma<bf16>::run(vf, pf, ws.o[dt]);
  }
}

template <typename T, int DH, int NTHR>
__global__ __launch_bounds__(NTHR) void attn_split_kernel(AttnArgs a) {
  constexpr int VEC = Mma<T>::VEC, KW = Mma<T>::KW;
  typedef typename Mma<T>::frag F;
  __shared__ AttnSmem<T, DH> sm;
  int sp, h, bc;
  split_coords(a, &sp, &h, &bc);
  const int b = bc / a.C;
  const int S = a.eff_ctx[b];
  const int s_lo = ctx_lo(S, a.window), kf0 = ctx_first(S, a.window) - s_lo;
  const int k_beg = s_lo + sp * a.split;
  if (sp > 0 && k_beg >= S) return;
  const int k_end = min(k_beg + a.split, S);
  const int group = a.hq / a.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const bool active = wave < group;  // spare waves only help staging
  const int head = h * group + (active ? wave : 0);

  // Q^T fragments (B operand): query row r16 of this head.
  F qf[DH / KW];
  const T *qrow = (const T *)a.q + ((long)bc * a.B + r16) * a.hq * DH + head * DH + VEC * g;
#pragma unroll
  for (int ks = 0; ks < DH / KW; ++ks)
    qf[ks] = (active && r16 < a.B) ? load_frag<T>(qrow + ks * KW) : zero_frag<T>();

  WaveState<T, DH> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c_log2 = a.scale * 1.4426950408889634f;  // score -> log2 units

  // chunks: the context range, then (split 0 only) the B block keys
  const int nctx = k_end > k_beg ? (k_end - k_beg + ATT_KC - 1) / ATT_KC : 0;
  const int nchunk = nctx + (sp == 0 ? 1 : 0);
  const T *kcache = (const T *)a.kc + ((long)b * a.hkv + h) * a.cap * DH;
  // V cache: tiles of ATT_KC keys, each tile d-major [DH][ATT_KC] and contiguous
  const T *vcache = (const T *)a.vc + ((long)b * a.hkv + h) * DH * a.cap;
  const T *kblock = (const T *)a.kb + (long)bc * a.B * a.hkv * DH + (long)h * DH;
  const T *vblock = (const T *)a.vb + ((long)bc * a.hkv + h) * DH * ATT_VBS;
  ChunkLoader<T, DH, NTHR> ld;
  auto issue = [&](int c) {
    if (c < nctx) {
      const int k0 = k_beg + c * ATT_KC;
      ld.load(kcache + (long)k0 * DH, DH, vcache + (long)k0 * DH, ATT_KC, min(ATT_KC, k_end - k0));
    } else {
      ld.load(kblock, (long)a.hkv * DH, vblock, ATT_VBS, a.B);
    }
  };
  issue(0);
  ld.store(sm, 0);
  __syncthreads();
  int nk = ld.nk;
  for (int c = 0; c < nchunk; ++c) {
    const int cur = c & 1;
    if (c + 1 < nchunk) issue(c + 1);
    // the window's first visible key lies in context chunk 0 of split 0
    const int kf = (sp == 0 && c == 0 && c < nctx) ? kf0 : 0;
    if (active) attend_chunk<T, DH, PadLayout<T, DH>>(sm.k[cur], sm.vt[cur], qf, nk, kf, c_log2, st);
    if (c + 1 < nchunk) {
      nk = ld.nk;
      ld.store(sm, cur ^ 1);
    }
    __syncthreads();
  }
  if (!active) return;

  // Row sum over the four lane groups, then the partial record.
  st.l += __shfl_xor(st.l, 16, WAVE);
  st.l += __shfl_xor(st.l, 32, WAVE);
  if (r16 < a.B) {
    const long rec = (((long)bc * a.hq + head) * a.nsplit + sp) * a.B + r16;
    float *op = a.opart + rec * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      *reinterpret_cast<f32x4 *>(op + dt * 16 + 4 * g) = st.o[dt];
    if (g == 0) {
      a.mlpart[rec * 2] = st.m * c_log2;  // running max in log2 units
      a.mlpart[rec * 2 + 1] = st.l;
    }
  }
}

// bf16 variant fed by direct global->LDS copies: the context chunks stream
// through a ring of ATT_NS buffers, ATT_NS - 1 chunks ahead of the waves
// (K and V^T of a cached chunk are each one contiguous block of 64 keys).
// A ring of two (64 KB at dh = 128) lets two workgroups share a compute
// unit, so one's start (Q load, first copy) and end (merge, partial record)
// overlap the other's streaming.
// Split 0 first takes its B block keys, staged through registers into the
// ring buffer the prologue leaves free.  A last chunk holding nk < 64 valid
// keys has its V^T columns nk..63 zeroed in LDS once its copies have landed,
// so whatever the cache holds beyond the context cannot reach P.V; its K rows
// are covered by the score mask.
constexpr int ATT_NS = 2;
static_assert(ATT_NS >= 2 && ATT_NS <= 4, "the wait ladder covers rings of 2 to 4");

template <int DH>
struct AttnRing {
  bf16 k[ATT_NS][ATT_KC * DH];
  bf16 vt[ATT_NS][DH * ATT_KC];
};

template <int DH, int NTHR, int KSPLIT>
__global__ __launch_bounds__(NTHR) void attn_split_dma_kernel(AttnArgs a) {
  using T = bf16;
  using Lay = SwzLayout<DH>;
  constexpr int VEC = Mma<T>::VEC, KW = Mma<T>::KW;
  constexpr int NWV = NTHR / 64;
  constexpr int CPK = ATT_KC * DH * 2 / 1024;  // copies per chunk, K (and V^T)
  constexpr int PER = CPK / NWV;               // copies per wave per chunk, each of K and V^T
  constexpr int OPS = 2 * PER;
  constexpr int KROWS = 1024 / (DH * 2);       // K rows per copy
  static_assert(CPK % NWV == 0, "copies must split evenly over the waves");
  typedef typename Mma<T>::frag F;
  __shared__ AttnRing<DH> sm;
  int sp, h, bc;
  split_coords(a, &sp, &h, &bc);
  const int b = bc / a.C;
  const int S = a.eff_ctx[b];
  const int s_lo = ctx_lo(S, a.window), kf0 = ctx_first(S, a.window) - s_lo;
  const int k_beg = s_lo + sp * a.split;
  if (sp > 0 && k_beg >= S) return;
  const int k_end = min(k_beg + a.split, S);
  const int group = a.hq / a.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  // KSPLIT = 2: wave set ks = wave / group takes keys 32 ks .. 32 ks + 31 of
  // every chunk with a softmax state of its own; the sets merge at the end
  const int kset = wave / group;
  const bool active = kset < KSPLIT;
  const int head = h * group + (active ? wave % group : 0);

  const int nctx = k_end > k_beg ? (k_end - k_beg + ATT_KC - 1) / ATT_KC : 0;
  const T *kcache = (const T *)a.kc + ((long)b * a.hkv + h) * a.cap * DH;
  const T *vcache = (const T *)a.vc + ((long)b * a.hkv + h) * DH * a.cap;
  // per-lane byte offsets of this wave's copies within a chunk: copy j of
  // wave w fills LDS bytes [1024 q, 1024 q + 1024), q = j * NWV + w
  uint32_t koff[PER], voff[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int q = j * NWV + wave;
    const int key = q * KROWS + lane / (DH / 8), kch = (lane % (DH / 8)) ^ Lay::kswz(key);
    koff[j] = (uint32_t)(key * DH * 2 + kch * 16);
    const int d = q * 8 + lane / 8, vch = (lane % 8) ^ Lay::vswz(d);
    voff[j] = (uint32_t)(d * ATT_KC * 2 + vch * 16);
  }
  auto issue = [&](int c) {
    const int k0 = k_beg + c * ATT_KC;
    const T *kb = kcache + (long)k0 * DH, *vb = vcache + (long)k0 * DH;
    const int slot = c % ATT_NS;
    const uint32_t kl = lds_u32(&sm.k[slot][0]), vl = lds_u32(&sm.vt[slot][0]);
#pragma unroll
    for (int j = 0; j < PER; ++j) dma16(kb, koff[j], kl + (j * NWV + wave) * 1024);
#pragma unroll
    for (int j = 0; j < PER; ++j) dma16(vb, voff[j], vl + (j * NWV + wave) * 1024);
  };
  // Q^T fragments (B operand): query row r16 of this head.  Their loads go
  // out just before the first ring copies and are covered by the loop's first
  // wait (vector-memory loads retire in issue order), so a workgroup's start
  // pays one memory round trip, not two (bs-32 attention 144.3 -> 143.9 us,
  // bs 4 x 32K 105.6 -> 105.1 us).  The compiler's own wait before their
  // first use is a full vmcnt(0), as it does not see the copies; with a ring
  // of two the loop waits for every copy at each chunk anyway.
  F qf[DH / KW];
  const T *qrow = (const T *)a.q + ((long)bc * a.B + r16) * a.hq * DH + head * DH + VEC * g;
#pragma unroll
  for (int ks = 0; ks < DH / KW; ++ks)
    qf[ks] = (active && r16 < a.B) ? load_frag<T>(qrow + ks * KW) : zero_frag<T>();
#pragma unroll
  for (int p = 0; p < ATT_NS - 1; ++p)
    if (p < nctx) issue(p);

  WaveState<T, DH> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c_log2 = a.scale * 1.4426950408889634f;  // score -> log2 units

  if (sp == 0) {
    // block keys -> ring buffer ATT_NS - 1: K rows 0..B-1, V^T columns 0..B-1,
    // every other V^T column zero
    constexpr int BS = ATT_NS - 1;
    const T *kblock = (const T *)a.kb + (long)bc * a.B * a.hkv * DH + (long)h * DH;
    const T *vblock = (const T *)a.vb + ((long)bc * a.hkv + h) * DH * ATT_VBS;
    char *kl = reinterpret_cast<char *>(&sm.k[BS][0]);
    char *vl = reinterpret_cast<char *>(&sm.vt[BS][0]);
    for (int i = threadIdx.x; i < a.B * (DH / 8); i += NTHR) {
      const int key = i / (DH / 8), ch = i % (DH / 8);
      *reinterpret_cast<F *>(kl + Lay::kbyte(key, ch)) =
          load_frag<T>(kblock + (long)key * a.hkv * DH + ch * 8);
    }
    for (int i = threadIdx.x; i < DH * (ATT_KC / 8); i += NTHR) {
      const int d = i / (ATT_KC / 8), ch = i % (ATT_KC / 8);
      F v = zero_frag<T>();
      if (ch * 8 < a.B) {  // ATT_VBS = 16 columns, the first B of them valid
        v = load_frag<T>(vblock + (long)d * ATT_VBS + ch * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (ch * 8 + e >= a.B) v[e] = T(0.0f);
      }
      *reinterpret_cast<F *>(vl + Lay::vbyte(d, ch)) = v;
    }
    __syncthreads();
    if (KSPLIT == 1) {
      if (active) attend_chunk<T, DH, Lay>(sm.k[BS], sm.vt[BS], qf, a.B, 0, c_log2, st);
    } else if (kset == 0) {  // B <= 16 keys: all in the first sub-chunk
      attend_sub<DH, Lay>(sm.k[BS], sm.vt[BS], qf, 0, a.B, 0, c_log2, st);
    }
  }

  for (int c = 0; c < nctx; ++c) {
    // this wave's copies of chunk c are done once at most the copies of the
    // chunks after it (up to ATT_NS - 2) are outstanding
    const int ahead = min(nctx - 1 - c, ATT_NS - 2);
    if (ATT_NS >= 4 && ahead >= 2) wait_vmcnt<2 * OPS>();
    else if (ATT_NS >= 3 && ahead >= 1) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    __syncthreads();  // every wave's copies visible; slot (c - 1) % ATT_NS free
    const int slot = c % ATT_NS;
    const int nk = min(ATT_KC, k_end - (k_beg + c * ATT_KC));
    if (nk < ATT_KC) {
      char *vl = reinterpret_cast<char *>(&sm.vt[slot][0]);
      for (int i = threadIdx.x; i < DH * (ATT_KC / 8); i += NTHR) {
        const int d = i / (ATT_KC / 8), ch = i % (ATT_KC / 8);
        if (ch * 8 + 8 <= nk) continue;
        F *p = reinterpret_cast<F *>(vl + Lay::vbyte(d, ch));
        F v = *p;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (ch * 8 + e >= nk) v[e] = T(0.0f);
        *p = v;
      }
      __syncthreads();
    }
    if (c + ATT_NS - 1 < nctx) issue(c + ATT_NS - 1);
    // the window's first visible key lies in chunk 0 of split 0; split 0 has
    // taken its block keys already, so a wave set whose sub-chunk is wholly
    // below the window keeps a finite reference
    const int kf = (sp == 0 && c == 0) ? kf0 : 0;
    if (KSPLIT == 1) {
      if (active) attend_chunk<T, DH, Lay>(sm.k[slot], sm.vt[slot], qf, nk, kf, c_log2, st);
    } else if (active) {
      const int nks = min(32, nk - 32 * kset);
      if (nks > 0)
        attend_sub<DH, Lay>(sm.k[slot], sm.vt[slot], qf, kset, nks, kf - 32 * kset, c_log2, st);
    }
  }
  if constexpr (KSPLIT == 2) {
    // set 1 hands its (m, l, O) to set 0 through the (now idle) ring: per
    // head and lane, 4 f32 of O per dh tile, then l and m
    constexpr int REC = DH / 4 + 4;  // floats per lane record (16-byte multiple)
    static_assert(NTHR / 64 / KSPLIT * 64 * REC * 4 <= (int)sizeof(AttnRing<DH>),
                  "merge staging must fit the ring");
    float *xs = reinterpret_cast<float *>(&sm) + (long)((wave % group) * 64 + lane) * REC;
    __syncthreads();
    if (kset == 1) {
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) *reinterpret_cast<f32x4 *>(xs + 4 * dt) = st.o[dt];
      xs[DH / 4] = st.l;
      xs[DH / 4 + 1] = st.m;
    }
    __syncthreads();
    if (kset != 0) return;
    const float m1 = xs[DH / 4 + 1];
    const float mm = fmaxf(st.m, m1);  // finite: set 0 always saw a key
    const float a0 = __builtin_amdgcn_exp2f((st.m - mm) * c_log2);
    const float a1 = __builtin_amdgcn_exp2f((m1 - mm) * c_log2);
    st.l = a0 * st.l + a1 * xs[DH / 4];
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      st.o[dt] = a0 * st.o[dt] + a1 * *reinterpret_cast<const f32x4 *>(xs + 4 * dt);
    st.m = mm;
  } else {
    __syncthreads();  // every wave is done with the ring before it stages records
  }
  if (!active) return;

  st.l += __shfl_xor(st.l, 16, WAVE);
  st.l += __shfl_xor(st.l, 32, WAVE);
  // The head's B records are one contiguous run of B * DH floats; a lane holds
  // 4 dims of one row, so the wave stages O as [16][DH + 4] floats in LDS
  // (within the region it used for the merge, or its own ring share) and
  // writes the run with 16-byte stores across consecutive dims.
  constexpr int OS = DH + 4, REGION = 64 * (DH / 4 + 4);  // floats: staged tile, wave's region
  static_assert(16 * OS <= REGION, "staging fits the wave's merge region");
  constexpr int STAGED_WAVES = KSPLIT == 2 ? NTHR / 128 : NTHR / 64;
  constexpr bool STAGE = STAGED_WAVES * REGION * 4 <= (int)sizeof(AttnRing<DH>);
  const long rec0 = (((long)bc * a.hq + head) * a.nsplit + sp) * a.B;
  float *op = a.opart + rec0 * DH;
  if constexpr (STAGE) {
    float *ost = reinterpret_cast<float *>(&sm) + (long)(KSPLIT == 2 ? wave % group : wave) * REGION;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      *reinterpret_cast<f32x4 *>(ost + r16 * OS + dt * 16 + 4 * g) = st.o[dt];
    for (int i = lane; i < a.B * (DH / 4); i += 64) {
      const int row = i / (DH / 4), c4 = 4 * (i % (DH / 4));
      *reinterpret_cast<f32x4 *>(op + (long)row * DH + c4) =
          *reinterpret_cast<const f32x4 *>(ost + row * OS + c4);
    }
  } else if (r16 < a.B) {
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      *reinterpret_cast<f32x4 *>(op + (long)r16 * DH + dt * 16 + 4 * g) = st.o[dt];
  }
  if (r16 < a.B && g == 0) {
    a.mlpart[(rec0 + r16) * 2] = st.m * c_log2;
    a.mlpart[(rec0 + r16) * 2 + 1] = st.l;
  }
}

// Merge the split partials: out = sum_s w_s O_s / sum_s w_s l_s with
// w_s = exp2(m_s - M), M the largest split max.  One workgroup per
// (sequence-copy, head, group of 512/dh query rows), one float4 of one row
// per thread; splits are merged in a fixed order.
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int bc = blockIdx.x, head = blockIdx.y;
  const int dh = a.dh, per_row = dh / 4, rows_per_wg = 128 / per_row;
  const int s = blockIdx.z * rows_per_wg + threadIdx.x / per_row;
  const int d = (threadIdx.x % per_row) * 4;
  if (s >= a.B) return;
  const int b = bc / a.C;
  const int S = a.eff_ctx[b] - ctx_lo(a.eff_ctx[b], a.window);  // keys from the first split
  const int nvalid = max(1, (S + a.split - 1) / a.split);
  const long rec0 = ((long)bc * a.hq + head) * a.nsplit * a.B + s;  // record of split sp: rec0 + sp*B
  // splits in groups of 8 with predicated loads, so a group's loads are in
  // flight together; the accumulation order is the split order
  constexpr int G = 8;
  float M = -INFINITY;
  for (int sp0 = 0; sp0 < nvalid; sp0 += G) {
    float mv[G];
#pragma unroll
    for (int i = 0; i < G; ++i)
      mv[i] = sp0 + i < nvalid ? a.mlpart[(rec0 + (long)(sp0 + i) * a.B) * 2] : -INFINITY;
#pragma unroll
    for (int i = 0; i < G; ++i) M = fmaxf(M, mv[i]);
  }
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < nvalid; sp0 += G) {
    float mv[G], lv[G];
    f32x4 ov[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const long r = rec0 + (long)(sp0 + i) * a.B;
      const bool ok = sp0 + i < nvalid;
      mv[i] = ok ? a.mlpart[r * 2] : -INFINITY;
      lv[i] = ok ? a.mlpart[r * 2 + 1] : 0.f;
      ov[i] = ok ? *reinterpret_cast<const f32x4 *>(a.opart + r * dh + d) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (sp0 + i >= nvalid) break;
      const float w = exp2f(mv[i] - M);
      L += w * lv[i];
      o += w * ov[i];
    }
  }
  const float inv = 1.0f / L;
  T *dst = (T *)a.out + ((long)bc * a.B + s) * a.hq * dh + (long)head * dh + d;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(o[e] * inv);
}

// The same merge for plans of more than 8 splits, in the same split order:
// the row's threads first load the (m, l) of different splits at once and
// take M by shuffles, the weights go through LDS, and the O vectors are then
// loaded 16 splits at a time: three dependent rounds of loads at 32 splits
// instead of eight.  (Up to 8 splits the kernel above needs two rounds and
// no barrier.)
constexpr int ATT_MAX_SPLITS = 128;  // the split plan's cap
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_wide_kernel(AttnArgs a) {
  constexpr int MAXR = 128 / 16;  // rows per workgroup at dh = 64
  __shared__ float sw[MAXR][ATT_MAX_SPLITS], sl[MAXR][ATT_MAX_SPLITS];
  const int bc = blockIdx.x, head = blockIdx.y;
  const int dh = a.dh, per_row = dh / 4, rows_per_wg = 128 / per_row;
  const int rw = threadIdx.x / per_row, j = threadIdx.x % per_row;
  const int s = blockIdx.z * rows_per_wg + rw;
  const int d = j * 4;
  const bool live = s < a.B;
  const int b = bc / a.C;
  const int S = a.eff_ctx[b] - ctx_lo(a.eff_ctx[b], a.window);  // keys from the first split
  const int nvalid = max(1, (S + a.split - 1) / a.split);
  const long rec0 = ((long)bc * a.hq + head) * a.nsplit * a.B + (live ? s : 0);  // + sp*B
  // lane j of a row takes splits j, j + per_row, ... (per_row >= 16 lanes)
  constexpr int SPL = ATT_MAX_SPLITS / 16;
  float mv[SPL], lv[SPL];
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int sp = j + i * per_row;
    const bool ok = live && sp < nvalid;
    const long r = rec0 + (long)sp * a.B;
    mv[i] = ok ? a.mlpart[r * 2] : -INFINITY;
    lv[i] = ok ? a.mlpart[r * 2 + 1] : 0.f;
    M = fmaxf(M, mv[i]);
  }
  // the row's lanes are an aligned group of per_row lanes of one wave
  for (int o = per_row / 2; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, WAVE));
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int sp = j + i * per_row;
    if (live && sp < nvalid) {
      sw[rw][sp] = exp2f(mv[i] - M);
      sl[rw][sp] = lv[i];
    }
  }
  __syncthreads();
  if (!live) return;
  constexpr int G = 16;
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < nvalid; sp0 += G) {
    f32x4 ov[G];
#pragma unroll
    for (int i = 0; i < G; ++i)
      ov[i] = sp0 + i < nvalid
                  ? *reinterpret_cast<const f32x4 *>(a.opart + (rec0 + (long)(sp0 + i) * a.B) * dh + d)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (sp0 + i >= nvalid) break;
      const float w = sw[rw][sp0 + i];
      L += w * sl[rw][sp0 + i];
      o += w * ov[i];
    }
  }
  const float inv = 1.0f / L;
  T *dst = (T *)a.out + ((long)bc * a.B + s) * a.hq * dh + (long)head * dh + d;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(o[e] * inv);
}

template <typename T, int DH, int NTHR>
static void launch_nthr(const AttnArgs &a, hipStream_t st) {
  const dim3 grid(a.nsplit * a.hkv * a.bs * a.C);
  hipLaunchKernelGGL((attn_split_kernel<T, DH, NTHR>), grid, dim3(NTHR), 0, st, a);
}

// Whether two wave sets of NTHR / 128 heads can merge through the ring.
template <int DH, int NTHR>
constexpr bool ksplit_fits() {
  return NTHR / 128 * 64 * (DH / 4 + 4) * 4 <= (int)sizeof(AttnRing<DH>);
}

template <int DH, int NTHR, int KSPLIT>
static void launch_dma(const AttnArgs &a, hipStream_t st) {
  const dim3 grid(a.nsplit * a.hkv * a.bs * a.C);
  hipLaunchKernelGGL((attn_split_dma_kernel<DH, NTHR, KSPLIT>), grid, dim3(NTHR), 0, st, a);
}

template <typename T, int DH>
static void launch_typed(const AttnArgs &a, hipStream_t st) {
  const int group = a.hq / a.hkv;
  if constexpr (std::is_same<T, bf16>::value) {
    // direct-copy ring; two wave sets per head while they fit in 1024 threads
    // and their merge fits the ring
    // (the K and V^T copies of a chunk must split evenly over the waves)
    constexpr int CPK = ATT_KC * DH * 2 / 1024;
    if (group <= 4) launch_dma<DH, 512, 2>(a, st);
    else if constexpr (CPK % 16 == 0) {
      if constexpr (ksplit_fits<DH, 1024>()) {
        if (group <= 8) launch_dma<DH, 1024, 2>(a, st);
        else launch_dma<DH, 1024, 1>(a, st);
      } else {
        launch_dma<DH, 1024, 1>(a, st);
      }
    } else {
      if (group <= 8) launch_nthr<T, DH, 512>(a, st);
      else launch_nthr<T, DH, 1024>(a, st);
    }
  } else {
    if (group <= 4) launch_nthr<T, DH, 256>(a, st);
    else if (group <= 8) launch_nthr<T, DH, 512>(a, st);
    else launch_nthr<T, DH, 1024>(a, st);
  }
  const int rows_per_wg = 128 / (a.dh / 4);
  const dim3 cgrid(a.bs * a.C, a.hq, (a.B + rows_per_wg - 1) / rows_per_wg);
  if (a.nsplit > 8) hipLaunchKernelGGL(attn_combine_wide_kernel<T>, cgrid, dim3(128), 0, st, a);
  else hipLaunchKernelGGL(attn_combine_kernel<T>, cgrid, dim3(128), 0, st, a);
}

void launch_attention_worklist(const AttnArgs &a, int *list, hipStream_t st) {
  if (a.bs * a.C == 0) return;
  hipLaunchKernelGGL(attn_worklist_kernel, dim3(1), dim3(1024), 0, st, a, list);
}

void launch_attention(const AttnArgs &a, hipStream_t st) {
  if (a.bs * a.C == 0) return;
  if (a.dtype == 1) {
    if (a.dh == 128) launch_typed<bf16, 128>(a, st);
    else launch_typed<bf16, 64>(a, st);
  } else {
    launch_typed<float, 64>(a, st);
  }
}

}  // namespace dstill
