// Non-causal block attention over the injected context (DFlash review,
// Method / Inference: K_i = [W^K H_t ; W^K H_d], V_i likewise, the block
// attending bidirectionally; DStill, Setup and notation: context strictly
// before the anchor).  Each query of copy c of sequence b attends
//   [cached K/V rows 0 .. S_b-1 ; the B block keys of copy c]
// with no mask (SPOT, Method: a copy sees the prefix and itself only),
// scaled by 1/sqrt(dh), through a softmax over all S_b + B keys.
//
// Work decomposition ("split context"): one workgroup per (split, kv head,
// sequence-copy).  Its `group` waves each own one query head of the GQA
// group, i.e. B <= 16 query rows (one 16-row MFMA tile).  The workgroup walks
// its context range in chunks of 64 keys staged in LDS (K row-major, V
// transposed), computes S^T = K Q^T and O^T = V^T P^T on the matrix cores and
// keeps an online softmax per query; split 0 also takes the block keys.  The
// partial (m, l, O) of every split is merged by attn_combine with the
// log-sum-exp rule, which reproduces the single softmax up to rounding.
//
// Lane layout (see Mma in common.hpp): in S^T, lane l holds query l % 16 and,
// with the key rows of each 32-key sub-chunk permuted so that tile t row
// 4g + i is key 8g + 4t + i, the 8 consecutive keys 8g .. 8g+7 (g = l / 16).
// Those 8 probabilities are exactly that lane's B fragment of P^T, and the
// matching A fragment of V^T is 8 consecutive keys of one transposed V row.
// bf16 probabilities go through P.V as a hi + lo pair of bf16 fragments, so
// the product keeps about 16 significant bits of P (fp32 accumulation).
// The row max/sum over a query's keys is then a reduction over the four lane
// groups: two xor-shuffles (16, 32).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dstill {

constexpr int ATT_KC = 64;  // keys per LDS chunk

template <typename T, int DH>
struct AttnSmem {
  static constexpr int VEC = Mma<T>::VEC;
  static constexpr int KS = DH + VEC;      // K row stride (elements), 16-byte pad
  static constexpr int VS = ATT_KC + VEC;  // V^T row stride
  T k[ATT_KC * KS];
  T vt[DH * VS];
};

// Stage `nk` keys (rows 0..nk-1 of src, row stride `stride` elements) into
// LDS; rows nk..63 are zero-filled so no stale value can reach P*V.
template <typename T, int DH>
__device__ __forceinline__ void stage_chunk(AttnSmem<T, DH> &sm, const T *__restrict__ ksrc,
                                            const T *__restrict__ vsrc, long stride, int nk) {
  constexpr int VEC = Mma<T>::VEC;
  constexpr int VPR = DH / VEC;  // vectors per row
  typedef typename Mma<T>::frag F;
  for (int idx = threadIdx.x; idx < ATT_KC * VPR; idx += blockDim.x) {
    const int key = idx / VPR, c = (idx % VPR) * VEC;
    F kv = zero_frag<T>(), vv = zero_frag<T>();
    if (key < nk) {
      kv = load_frag<T>(ksrc + key * stride + c);
      vv = load_frag<T>(vsrc + key * stride + c);
    }
    *reinterpret_cast<F *>(&sm.k[key * AttnSmem<T, DH>::KS + c]) = kv;
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm.vt[(c + e) * AttnSmem<T, DH>::VS + key] = vv[e];
  }
}

template <typename T, int DH>
struct WaveState {
  float m, l;
  f32x4 o[DH / 16];
};

// One wave's pass over a staged chunk holding `nk` valid keys.
template <typename T, int DH>
__device__ __forceinline__ void attend_chunk(const AttnSmem<T, DH> &sm,
                                             const typename Mma<T>::frag *qf, int nk,
                                             float scale_log2, WaveState<T, DH> &ws) {
  constexpr int VEC = Mma<T>::VEC, KW = Mma<T>::KW;
  typedef typename Mma<T>::frag F;
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  for (int sc = 0; sc * 32 < nk; ++sc) {
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int krow = sc * 32 + 8 * (r16 >> 2) + 4 * t + (r16 & 3);
      const T *kp = &sm.k[krow * AttnSmem<T, DH>::KS + VEC * g];
#pragma unroll
      for (int ks = 0; ks < DH / KW; ++ks)
        s[t] = Mma<T>::run(*reinterpret_cast<const F *>(kp + ks * KW), qf[ks], s[t]);
    }
    float p[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = sc * 32 + 8 * g + 4 * t + i;
        const float v = key < nk ? s[t][i] * scale_log2 : -INFINITY;
        p[4 * t + i] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, WAVE));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, WAVE));
    const float mnew = fmaxf(ws.m, cmax);
    const float alpha = exp2f(ws.m - mnew);
    ws.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) ws.o[dt] *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(p[e] - mnew);
      ws.l += p[e];
    }
    ws.m = mnew;
    // P^T fragments: bf16 packs all 8 keys in one fragment; fp32 uses two.
    // In bf16 the probabilities are carried as a hi + lo pair (lo = the
    // rounding residual of hi), so P.V keeps ~16 significant bits of P.
    constexpr int NPF = 8 / VEC;
    constexpr bool SPLIT = VEC == 8;
    F pf[NPF], pl[NPF];
#pragma unroll
    for (int f = 0; f < NPF; ++f)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const T hi = from_f32<T>(p[f * VEC + e]);
        pf[f][e] = hi;
        if (SPLIT) pl[f][e] = from_f32<T>(p[f * VEC + e] - to_f32(hi));
      }
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const T *vp = &sm.vt[(dt * 16 + r16) * AttnSmem<T, DH>::VS + sc * 32 + 8 * g];
#pragma unroll
      for (int f = 0; f < NPF; ++f) {
        const F vf = *reinterpret_cast<const F *>(vp + f * VEC);
        ws.o[dt] = Mma<T>::run(vf, pf[f], ws.o[dt]);
        if (SPLIT) ws.o[dt] = Mma<T>::run(vf, pl[f], ws.o[dt]);
      }
    }
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(1024) void attn_split_kernel(AttnArgs a) {
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
  const int head = h * group + wave;

  // Q^T fragments (B operand): query row r16 of this head.
  F qf[DH / KW];
  const T *qrow = (const T *)a.q + ((long)bc * a.B + r16) * a.hq * DH + head * DH + VEC * g;
#pragma unroll
  for (int ks = 0; ks < DH / KW; ++ks)
    qf[ks] = r16 < a.B ? load_frag<T>(qrow + ks * KW) : zero_frag<T>();

  WaveState<T, DH> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float scale_log2 = a.scale * 1.4426950408889634f;

  const long cache_row0 = ((long)b * a.hkv + h) * a.cap;
  for (int k0 = k_beg; k0 < k_end; k0 += ATT_KC) {
    const int nk = min(ATT_KC, k_end - k0);
    __syncthreads();
    stage_chunk<T, DH>(sm, (const T *)a.kc + (cache_row0 + k0) * DH,
                       (const T *)a.vc + (cache_row0 + k0) * DH, DH, nk);
    __syncthreads();
    attend_chunk<T, DH>(sm, qf, nk, scale_log2, st);
  }
  if (sp == 0) {
    const long boff = ((long)bc * a.B) * a.hkv * DH + (long)h * DH;
    __syncthreads();
    stage_chunk<T, DH>(sm, (const T *)a.kb + boff, (const T *)a.vb + boff, (long)a.hkv * DH, a.B);
    __syncthreads();
    attend_chunk<T, DH>(sm, qf, a.B, scale_log2, st);
  }

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
      a.mlpart[rec * 2] = st.m;
      a.mlpart[rec * 2 + 1] = st.l;
    }
  }
}

// Merge the split partials of one (sequence-copy, head): weights
// exp2(m_s - M) / L with L = sum_s exp2(m_s - M) l_s, computed once per query
// row into LDS, then a weighted sum of the split outputs, 4 values per thread.
constexpr int COMBINE_MAX_SPLITS = 128;

template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  __shared__ float wts[16][COMBINE_MAX_SPLITS];
  const int bc = blockIdx.x, head = blockIdx.y;
  const int b = bc / a.C;
  const int S = a.eff_ctx[b];
  const int nvalid = max(1, (S + a.split - 1) / a.split);
  const int dh = a.dh;
  const long rec0 = ((long)bc * a.hq + head) * a.nsplit * a.B;  // record (sp, s) = rec0 + sp*B + s
  for (int s = threadIdx.x; s < a.B; s += blockDim.x) {
    float M = -INFINITY;
    for (int sp = 0; sp < nvalid; ++sp) M = fmaxf(M, a.mlpart[(rec0 + (long)sp * a.B + s) * 2]);
    float L = 0.f;
    for (int sp = 0; sp < nvalid; ++sp) {
      const long r = rec0 + (long)sp * a.B + s;
      const float w = exp2f(a.mlpart[r * 2] - M);
      wts[s][sp] = w;
      L += w * a.mlpart[r * 2 + 1];
    }
    const float inv = 1.0f / L;
    for (int sp = 0; sp < nvalid; ++sp) wts[s][sp] *= inv;
  }
  __syncthreads();
  const int nv4 = dh / 4;
  for (int idx = threadIdx.x; idx < a.B * nv4; idx += blockDim.x) {
    const int s = idx / nv4, d = (idx % nv4) * 4;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < nvalid; ++sp)
      o += wts[s][sp] * *reinterpret_cast<const f32x4 *>(a.opart + (rec0 + (long)sp * a.B + s) * dh + d);
    T *dst = (T *)a.out + ((long)bc * a.B + s) * a.hq * dh + (long)head * dh + d;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(o[e]);
  }
}

template <typename T, int DH>
static void launch_typed(const AttnArgs &a, hipStream_t st) {
  const int group = a.hq / a.hkv;
  dim3 grid(a.nsplit, a.hkv, a.bs * a.C);
  hipLaunchKernelGGL((attn_split_kernel<T, DH>), grid, dim3(64 * group), 0, st, a);
  hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(a.bs * a.C, a.hq), dim3(256), 0, st, a);
}

void launch_attention(const AttnArgs &a, hipStream_t st) {
  if (a.bs * a.C == 0) return;
  if (a.dtype == 1) {
    if (a.dh == 128) launch_typed<bf16, 128>(a, st);
    else launch_typed<bf16, 64>(a, st);
  } else {
    if (a.dh == 128) launch_typed<float, 128>(a, st);
    else launch_typed<float, 64>(a, st);
  }
}

}  // namespace dstill
