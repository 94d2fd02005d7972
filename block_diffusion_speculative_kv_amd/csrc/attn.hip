// Non-causal block attention over the injected context (DFlash review,
// Method / Inference: K_i = [W^K H_t ; W^K H_d], V_i likewise, the block
// attending bidirectionally; DStill, Setup and notation: context strictly
// before the anchor).  Each query of copy c of sequence b attends
//   [cached K/V rows 0 .. S_b-1 ; the B block keys of copy c]
// with no mask (SPOT, Method: a copy sees the prefix and itself only),
// scaled by 1/sqrt(dh), through a softmax over all S_b + B keys.
//
// Work decomposition ("split context"): one workgroup per (split, kv head,
// sequence-copy).  Its first `group` waves each own one query head of the GQA
// group, i.e. B <= 16 query rows (one 16-row MFMA tile).  The workgroup walks
// its context range in chunks of 64 keys, computes S^T = K Q^T and
// O^T = V^T P^T on the matrix cores and keeps an online softmax per query;
// split 0 also takes the block keys.  Chunks are pipelined: the next chunk's
// K and V^T are loaded into registers while the waves work on the current
// one out of LDS, then written to the other LDS buffer (one barrier per
// chunk).  The V cache is stored in tiles of 64 keys, each d-major
// ([cap/64][dh][64] per sequence and head), so V^T of a chunk is one
// contiguous 16 KB block, like the chunk of K.  The
// partial (m, l, O) of every split is merged by attn_combine with the
// log-sum-exp rule, which reproduces the single softmax up to rounding.
//
// Lane layout (see Mma in common.hpp): in S^T, lane l holds query l % 16 and,
// with the key rows of each 32-key sub-chunk permuted so that tile t row
// 4g + i is key 8g + 4t + i, the 8 consecutive keys 8g .. 8g+7 (g = l / 16).
// Those 8 probabilities are exactly that lane's B fragment of P^T, and the
// matching A fragment of V^T is 8 consecutive keys of one V^T row.  The row
// max/sum over a query's keys is then a reduction over the four lane
// groups: two xor-shuffles (16, 32).
#include <math.h>

#include "common.hpp"
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

template <typename T, int DH>
struct WaveState {
  float m, l;
  f32x4 o[DH / 16];
};

// One wave's pass over a staged chunk holding `nk` valid keys (1..64), with
// one online-softmax update for the whole chunk.  Scores stay in raw units
// (m is the running max of raw scores); probabilities are
// exp2(s * c - m * c) with c = log2(e) / sqrt(dh), one FMA and one v_exp_f32
// each.  The accumulators are rescaled only when some query's max grows
// (a wave-uniform branch), which after the first chunks is rare.
template <typename T, int DH>
__device__ __forceinline__ void attend_chunk(const T *__restrict__ ks_lds,
                                             const T *__restrict__ vt_lds,
                                             const typename Mma<T>::frag *qf, int nk, float c,
                                             WaveState<T, DH> &ws) {
  constexpr int VEC = Mma<T>::VEC, KW = Mma<T>::KW;
  constexpr int KS = AttnSmem<T, DH>::KS, VS = AttnSmem<T, DH>::VS;
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
      const T *kp = ks_lds + krow * KS + VEC * g;
#pragma unroll
      for (int ks = 0; ks < DH / KW; ++ks)
        s[t] = Mma<T>::run(*reinterpret_cast<const F *>(kp + ks * KW), qf[ks], s[t]);
    }
  }
  if (nk < ATT_KC) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (32 * (t >> 1) + 8 * g + 4 * (t & 1) + i >= nk) s[t][i] = -INFINITY;
  }
  float cmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  cmax = fmaxf(cmax, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                           fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 16, WAVE));
  cmax = fmaxf(cmax, __shfl_xor(cmax, 32, WAVE));
  const float mnew = fmaxf(ws.m, cmax);
  if (__any(mnew > ws.m)) {
    const float alpha = __builtin_amdgcn_exp2f((ws.m - mnew) * c);
    ws.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) ws.o[dt] *= alpha;
  }
  ws.m = mnew;
  const float mc = mnew * c;
  float p[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[t][i] = __builtin_amdgcn_exp2f(fmaf(s[t][i], c, -mc));
      ws.l += p[t][i];
    }
  // P^T fragments per sub-chunk: keys 8g .. 8g+7 are p[2sc][0..3], p[2sc+1][0..3].
  // bf16 carries them as a hi + lo pair (lo = the rounding residual of hi) so
  // P.V keeps ~16 significant bits of P; fp32 uses two exact fragments.
  constexpr int NPF = 8 / VEC;
  constexpr bool SPLIT = VEC == 8;
#pragma unroll
  for (int sc = 0; sc < 2; ++sc) {
    if (sc >= nsub) break;
    F pf[NPF], pl[NPF];
#pragma unroll
    for (int f = 0; f < NPF; ++f)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int k8 = f * VEC + e;  // 0..7
        const float pv = p[2 * sc + (k8 >> 2)][k8 & 3];
        const T hi = from_f32<T>(pv);
        pf[f][e] = hi;
        if (SPLIT) pl[f][e] = from_f32<T>(pv - to_f32(hi));
      }
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const T *vp = vt_lds + (dt * 16 + r16) * VS + sc * 32 + 8 * g;
#pragma unroll
      for (int f = 0; f < NPF; ++f) {
        const F vf = *reinterpret_cast<const F *>(vp + f * VEC);
        ws.o[dt] = Mma<T>::run(vf, pf[f], ws.o[dt]);
        if (SPLIT) ws.o[dt] = Mma<T>::run(vf, pl[f], ws.o[dt]);
      }
    }
  }
}

template <typename T, int DH, int NTHR>
__global__ __launch_bounds__(NTHR) void attn_split_kernel(AttnArgs a) {
  constexpr int VEC = Mma<T>::VEC, KW = Mma<T>::KW;
  typedef typename Mma<T>::frag F;
  __shared__ AttnSmem<T, DH> sm;
  const int sp = blockIdx.x, h = blockIdx.y, bc = blockIdx.z;
  const int b = bc / a.C;
  const int S = a.eff_ctx[b];
  const int k_beg = sp * a.split;
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
    if (active) attend_chunk<T, DH>(sm.k[cur], sm.vt[cur], qf, nk, c_log2, st);
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
  const int S = a.eff_ctx[b];
  const int nvalid = max(1, (S + a.split - 1) / a.split);
  const long rec0 = ((long)bc * a.hq + head) * a.nsplit * a.B + s;  // record of split sp: rec0 + sp*B
  float M = -INFINITY;
  for (int sp = 0; sp < nvalid; ++sp) M = fmaxf(M, a.mlpart[(rec0 + (long)sp * a.B) * 2]);
  float L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < nvalid; ++sp) {
    const long r = rec0 + (long)sp * a.B;
    const float w = exp2f(a.mlpart[r * 2] - M);
    L += w * a.mlpart[r * 2 + 1];
    o += w * *reinterpret_cast<const f32x4 *>(a.opart + r * dh + d);
  }
  const float inv = 1.0f / L;
  T *dst = (T *)a.out + ((long)bc * a.B + s) * a.hq * dh + (long)head * dh + d;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(o[e] * inv);
}

template <typename T, int DH, int NTHR>
static void launch_nthr(const AttnArgs &a, hipStream_t st) {
  dim3 grid(a.nsplit, a.hkv, a.bs * a.C);
  hipLaunchKernelGGL((attn_split_kernel<T, DH, NTHR>), grid, dim3(NTHR), 0, st, a);
}

template <typename T, int DH>
static void launch_typed(const AttnArgs &a, hipStream_t st) {
  const int group = a.hq / a.hkv;
  if (group <= 4) launch_nthr<T, DH, 256>(a, st);
  else if (group <= 8) launch_nthr<T, DH, 512>(a, st);
  else launch_nthr<T, DH, 1024>(a, st);
  const int rows_per_wg = 128 / (a.dh / 4);
  hipLaunchKernelGGL(attn_combine_kernel<T>,
                     dim3(a.bs * a.C, a.hq, (a.B + rows_per_wg - 1) / rows_per_wg), dim3(128), 0,
                     st, a);
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
