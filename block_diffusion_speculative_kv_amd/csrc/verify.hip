// Verification of a drafted block against the target's logits (DStill,
// Inference: greedy verification and the standard rejection-sampling
// verifier, a correction token after a rejection and a bonus token after
// full acceptance; DFlash review, Preliminary: tau = accepted + 1 in
// [1, gamma+1]).  The acceptance test and the residual are the textbook ones
// of speculative sampling (Leviathan et al.; Chen et al., both cited there):
// accept y ~ q_k while u_k < p_k(y) / q_k(y); at the first rejection draw from
// norm(max(0, p_k - q_k)); after gamma acceptances draw from p_gamma.  Draws
// use Gumbel-max over log-weights with counter-based Philox noise.
//
// Four kernels, all streaming:
//   vrow     per (target row, vocab split): greedy: max, argmax (lowest
//            id) and runner-up; rejection sampling: the softmax mass at
//            temperature T (fp64 accumulation)
//   vdecide  per sequence: merge the splits, then the greedy prefix match or
//            the accept scan (one lane per block slot, first failure by
//            ballot); writes the accepted prefix, tau and the flags
//   vsample  (rejection sampling) per (sequence, vocab split): Gumbel-max
//            over log max(0, p - q) of the rejected row, or over log p of
//            the bonus row, in fp64
//   vfinish  per sequence: merge and write the final token
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dstill {

struct VRowPart {
  float best, second;
  int idx, bad;
  float m, pad;
  double s;  // sum exp(z/T - m)
};

struct D2 {
  double best, second;
  int idx;
};
__device__ __forceinline__ void d2_push(D2 &a, double s, int i) {
  if (s > a.best || (s == a.best && i < a.idx)) {
    a.second = fmax(a.second, a.best);
    a.best = s;
    a.idx = i;
  } else {
    a.second = fmax(a.second, s);
  }
}
__device__ __forceinline__ D2 d2_merge(D2 a, D2 b) {
  if (b.best > a.best || (b.best == a.best && b.idx < a.idx)) {
    D2 t = a; a = b; b = t;
  }
  a.second = fmax(a.second, b.best);
  return a;
}

struct VSampPart {
  double best_r, second_r, best_p, second_p;
  int idx_r, idx_p, any_r, bad;
};

struct VerifyWs {
  VRowPart *rowpart;   // [bs*(gamma+1)][nsplit]
  double *lse_t;       // [bs*(gamma+1)]
  int *kstar;          // [bs]
  VSampPart *samp;     // [bs][nsamp]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline VerifyWs carve(void *ws, int bs, int gamma, int nsplit) {
  // (the sampling records come last, so their count does not move the rest)
  char *p = (char *)ws;
  VerifyWs w;
  const size_t rows = (size_t)bs * (gamma + 1);
  w.rowpart = (VRowPart *)p;
  p += align256(rows * nsplit * sizeof(VRowPart));
  w.lse_t = (double *)p;
  p += align256(rows * sizeof(double));
  w.kstar = (int *)p;
  p += align256((size_t)bs * sizeof(int));
  w.samp = (VSampPart *)p;
  return w;
}

size_t verify_ws_bytes(int bs, int gamma, int nsplit, int nsamp) {
  const size_t rows = (size_t)bs * (gamma + 1);
  return align256(rows * nsplit * sizeof(VRowPart)) + align256(rows * sizeof(double)) +
         align256((size_t)bs * sizeof(int)) + align256((size_t)bs * nsamp * sizeof(VSampPart));
}

int verify_plan_splits(int rows_, int vocab) {
  // about 1024 workgroups over the rows, at least 2048 ids each, at most 64
  const long rows = rows_ < 1 ? 1 : rows_;
  long n = (1024 + rows - 1) / rows;
  const long most = (vocab + 2047) / 2048;
  if (n > most) n = most;
  if (n > 64) n = 64;
  return n < 1 ? 1 : (int)n;
}

__device__ __forceinline__ int split_chunk(int vocab, int nsplit) {
  const int c = (vocab + nsplit - 1) / nsplit;
  return (c + 7) & ~7;
}

// Eight consecutive logits starting at p (16-byte aligned for bf16 rows of
// length % 8 == 0, two 16-byte loads for fp32).
__device__ __forceinline__ void ld8(const bf16 *p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
}
__device__ __forceinline__ void ld8(const float *p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

__device__ __forceinline__ float ld(const float *p, long i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16 *p, long i) { return static_cast<float>(p[i]); }

// ---- per-row statistics --------------------------------------------------
// Headroom of the lazy softmax reference in the row pass: terms are at most
// e^16, so a split's sums stay far inside fp32 (per group) and fp64 range.
constexpr float VROW_LAZY = 16.f;

template <typename TT>
__global__ __launch_bounds__(256) void vrow_kernel(VerifyArgs a, VerifyWs w) {
  __shared__ VRowPart red[4];
  const int row = blockIdx.x, sp = blockIdx.y;
  const int V = a.vocab;
  const int chunk = split_chunk(V, a.nsplit);
  const int v0 = sp * chunk, v1 = min(v0 + chunk, V);
  const TT *z = (const TT *)a.target + (long)row * V;
  const float invT = 1.0f / a.temperature;
  ArgTop2 arg;
  arg.best = -INFINITY;
  arg.second = -INFINITY;
  arg.idx = 0x7fffffff;
  float m = -INFINITY;
  double s = 0.0;
  int bad = 0;
  auto push = [&](float x, int v) {
    if (!isfinite(x)) { bad = 1; return; }
    top2_push(arg, x, v);
    const float y = x * invT;
    if (y > m) {
      s = s * exp((double)m - (double)y) + 1.0;
      m = y;
    } else {
      s += (double)expf(y - m);
    }
  };
  if ((V & 7) == 0) {
    // 8 consecutive ids per thread per step (v0 and v1 are multiples of 8):
    // the softmax reference moves at most once per group (one fp64
    // rescale, and only past the lazy headroom), the 8 terms exp(y - m) <=
    // e^VROW_LAZY are summed in fp32 with the hardware exp2 and folded into
    // the fp64 sum once
    // U groups per thread are loaded before any is reduced (more loads in
    // flight); each thread still takes its groups in increasing order.  One
    // top-2 per group position (8 independent chains instead of one); the
    // top-2 merge with lowest-id ties is order-independent.  Batches whose
    // values are all finite take a path without per-element branches.
    constexpr int U = 4;
    const int step = 8 * blockDim.x;
    ArgTop2 ag[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[e] = ArgTop2{-INFINITY, -INFINITY, 0x7fffffff};
    // (each position chain sees its ids in increasing order: top2_push_inc)
    // greedy decisions use the top-2 only, the rejection-sampling test the
    // softmax mass only (the flags for non-finite values come from either)
    const bool want_lse = a.mode != 0;
    auto group = [&](const float (&x)[8], int v) {
      if (!want_lse) {
#pragma unroll
        for (int e = 0; e < 8; ++e) top2_push_inc(ag[e], x[e], v + e);
        return;
      }
      float y[8], gm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = x[e] * invT;
        gm = fmaxf(gm, y[e]);
      }
      // Lazy reference: s holds sum exp(y - m) for a reference m that is
      // moved (with an fp64 rescale) only when a group's maximum exceeds it
      // by more than VROW_LAZY, so every term stays at most e^VROW_LAZY.
      // Moving it at every new maximum would run the fp64 exponential for
      // nearly every group of a wave (some lane almost always sees one).
      if (gm > m + VROW_LAZY) {
        s = (m == -INFINITY) ? 0.0 : s * exp((double)m - (double)gm);
        m = gm;
      }
      const float mc = m * 1.4426950408889634f;
      float s8 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s8 += __builtin_amdgcn_exp2f(fmaf(y[e], 1.4426950408889634f, -mc));
      s += (double)s8;
    };
    // x * 0 is 0 for finite x and NaN otherwise: one multiply-add per value
    // tells whether a batch holds a non-finite value
    auto all_finite = [](const float *x, int n) {
      float t = 0.f;
      for (int e = 0; e < n; ++e) t = fmaf(x[e], 0.f, t);
      return t == 0.f;
    };
    int vb = v0 + 8 * threadIdx.x;
    for (; vb + (U - 1) * step < v1; vb += U * step) {
      float xs[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) ld8(z + vb + u * step, xs[u]);
      if (all_finite(&xs[0][0], U * 8)) {
#pragma unroll
        for (int u = 0; u < U; ++u) group(xs[u], vb + u * step);
      } else {  // rare: element by element, skipping (and flagging) non-finite ones
        for (int u = 0; u < U; ++u)
          for (int e = 0; e < 8; ++e) push(xs[u][e], vb + u * step + e);
      }
    }
    for (; vb < v1; vb += step) {
      float x[8];
      ld8(z + vb, x);
      if (all_finite(x, 8)) {
        group(x, vb);
      } else {
        for (int e = 0; e < 8; ++e) push(x[e], vb + e);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) arg = top2_merge(arg, ag[e]);
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += blockDim.x) push(ld(z, v), v);
  }
  // wave merge
  for (int o = 32; o > 0; o >>= 1) {
    arg = top2_shfl_xor(arg, o);
    const float m2 = __shfl_xor(m, o, WAVE);
    const double s2 = __shfl_xor(s, o, WAVE);
    bad |= __shfl_xor(bad, o, WAVE);
    if (m2 != -INFINITY) {
      if (m == -INFINITY) { m = m2; s = s2; }
      else {
        const float M = fmaxf(m, m2);
        s = s * exp((double)m - M) + s2 * exp((double)m2 - M);
        m = M;
      }
    }
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    VRowPart p;
    p.best = arg.best; p.second = arg.second; p.idx = arg.idx; p.bad = bad;
    p.m = m; p.pad = 0.f; p.s = s;
    red[wave] = p;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    VRowPart t = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) {
      const VRowPart u = red[i];
      ArgTop2 x{t.best, t.second, t.idx}, y{u.best, u.second, u.idx};
      x = top2_merge(x, y);
      t.best = x.best; t.second = x.second; t.idx = x.idx;
      t.bad |= u.bad;
      if (u.m != -INFINITY) {
        if (t.m == -INFINITY) { t.m = u.m; t.s = u.s; }
        else {
          const float M = fmaxf(t.m, u.m);
          t.s = t.s * exp((double)t.m - M) + u.s * exp((double)u.m - M);
          t.m = M;
        }
      }
    }
    w.rowpart[(long)row * a.nsplit + sp] = t;
  }
}

// ---- decision scan ---------------------------------------------------------
template <typename TT>
__global__ __launch_bounds__(1024) void vdecide_kernel(VerifyArgs a, VerifyWs w) {
  struct RowRes {
    ArgTop2 arg;
    int bad;
    double lse;
  };
  __shared__ RowRes res[64];
  const int b = blockIdx.x, G = a.gamma, V = a.vocab;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  // Wave 0's per-slot inputs (lane k: the draft id, and for rejection
  // sampling the target and draft logits at it and the draft's log-sum-exp)
  // do not depend on the row merge: their loads are issued first.
  const int k = lane;
  int y = 0, yraw = 0;
  double zt_y = 0.0, zd_y = 0.0;
  float dl = 0.f;
  if (wave == 0 && k < G) {
    yraw = a.draft_ids[(long)b * G + k];
    y = yraw < 0 ? 0 : (yraw >= V ? V - 1 : yraw);
    if (a.mode != 0) {
      zt_y = (double)ld((const TT *)a.target, ((long)b * (G + 1) + k) * V + y);
      zd_y = (double)a.draft_logits[((long)b * G + k) * V + y];
      dl = a.draft_lse[(long)b * G + k];
    }
  }
  // Row merge, one wave per target row, lanes over the row's vocabulary
  // splits: top-2 and flags by wave reduction, then the log-sum-exp as
  // M + log(sum_j s_j exp(m_j - M)) with M the largest split maximum.
  for (int kr = wave; kr <= G; kr += nw) {
    const long row = (long)b * (G + 1) + kr;
    ArgTop2 arg{-INFINITY, -INFINITY, 0x7fffffff};
    float m = -INFINITY;
    double sv = 0.0;
    int bad = 0;
    for (int sp = lane; sp < a.nsplit; sp += WAVE) {
      const VRowPart p = w.rowpart[row * a.nsplit + sp];
      arg = top2_merge(arg, ArgTop2{p.best, p.second, p.idx});
      bad |= p.bad;
      if (p.m != -INFINITY) {
        if (m == -INFINITY) { m = p.m; sv = p.s; }
        else {
          const float M = fmaxf(m, p.m);
          sv = sv * exp((double)m - M) + p.s * exp((double)p.m - M);
          m = M;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      arg = top2_shfl_xor(arg, o);
      bad |= __shfl_xor(bad, o, WAVE);
    }
    const float M = wave_max(m);
    const double part = m == -INFINITY ? 0.0 : sv * exp((double)m - (double)M);
    const double S = wave_sum(part);
    if (lane == 0) {
      const double lse = (double)M + log(S);
      res[kr] = RowRes{arg, bad, lse};
      w.lse_t[row] = lse;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const bool rowlane = k <= G;
  ArgTop2 arg{-INFINITY, -INFINITY, 0x7fffffff};
  int bad = 0;
  double lse = 0.0;
  if (rowlane) {
    arg = res[k].arg;
    bad = res[k].bad;
    lse = res[k].lse;
  }
  if (k < G && y != yraw) bad = 1;
  uint32_t flags = 0;
  bool ok = false;  // slot k passes its test
  bool near = false;
  if (a.mode == 0) {
    ok = k < G && yraw == arg.idx;
    near = rowlane && (arg.best - arg.second) < NEAR_BAND;
  } else if (k < G) {
    const double T = (double)a.temperature;
    const double lp = zt_y / T - lse;
    const double lq = zd_y / T - (double)dl;
    const double ratio = exp(lp - lq);
    uint32_t raw[8];
    philox_block8(a.seed, 1u, (uint64_t)b, (uint64_t)k, a.cycle, 0, raw);
    const double u = (double)u24(raw[0]);
    ok = u < ratio;
    near = fabs(ratio - u) < (double)NEAR_BAND;
    if (!isfinite(zd_y) || !isfinite(dl)) bad = 1;
  }
  // first failing slot (gamma if all pass)
  const unsigned long long fail = __ballot(k < G && !ok);
  const int L = fail ? min(__builtin_ctzll(fail), G) : G;
  const unsigned long long bads = __ballot(bad != 0);
  if (bads) flags |= 16u;
  if (a.mode == 0) {
    if (__ballot(near && k <= L)) flags |= 1u;
  } else {
    if (__ballot(near && k <= L && k < G)) flags |= 2u;
  }
  // tokens: accepted prefix; slot L gets the target's token (greedy) or is
  // filled by vfinish (rejection sampling)
  if (k <= G) {
    int tok = -1;
    if (k < L) tok = y;
    else if (k == L && a.mode == 0) tok = arg.idx;
    if (!(k == L && a.mode != 0)) a.tokens[(long)b * (G + 1) + k] = tok;
  }
  if (k == 0) {
    a.tau[b] = L + 1;
    a.flags[b] = flags;
    w.kstar[b] = L;
  }
}

// ---- residual / bonus draw ---------------------------------------------------
// Per (sequence, vocabulary split): the bonus / fallback draw argmax (lp + g)
// over every id (lp = z_t / T - lse_t, g the Gumbel noise), and the residual
// draw argmax (log max(0, p - q) + g).  Since max(0, p - q) <= p, the
// residual score of an id is at most its bound lp + g.  The split is taken
// in windows of VS_GPT groups of 8 ids per thread; a first pass draws every
// id's noise and keeps, in registers, its fp32 bound and its fp32 noise
// (exact: the noise is an fp32 value).  With U the window's largest bound,
// ids are then evaluated exactly in fp64 (bound and, for a rejected row, the
// residual: two exponentials and a logarithm) in rounds: those with bound
// >= U - 4 first, then down to U - 16, then all the rest.  The first round
// holds the largest lp + g and every id within the near-tie band of it, so
// the bonus / fallback top-2 taken over the evaluated ids decides exactly
// what the full one does (the runner-up is used only against the band).
// The residual walk stops as soon as its best score lies the band (plus a
// rounding margin) above the current threshold: no id left out can then
// win, nor come within the band of the winner.  A block whose residual is
// empty (p <= q everywhere) evaluates every id.
constexpr int VS_GPT = 3;
constexpr int VS_THREADS = 256;

__device__ __forceinline__ double block_max_d(double v, double *sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, WAVE));
  __syncthreads();  // sh is free (earlier readers are done)
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = sh[0];
  for (int i = 1; i < VS_THREADS / 64; ++i) r = fmax(r, sh[i]);
  return r;
}

template <typename TT>
__global__ __launch_bounds__(VS_THREADS) void vsample_kernel(VerifyArgs a, VerifyWs w) {
  __shared__ VSampPart red[VS_THREADS / 64];
  __shared__ double shd[VS_THREADS / 64];
  const int b = blockIdx.x, sp = blockIdx.y;
  const int G = a.gamma, V = a.vocab;
  const int ks = w.kstar[b];
  const long trow = (long)b * (G + 1) + ks;
  const double lse_t = w.lse_t[trow];
  const bool bonus = ks >= G;
  const double lse_d = bonus ? 0.0 : (double)a.draft_lse[(long)b * G + ks];
  const TT *zt = (const TT *)a.target + trow * V;
  const float *zd = bonus ? nullptr : a.draft_logits + ((long)b * G + ks) * V;
  const double T = (double)a.temperature;
  const int chunk = split_chunk(V, a.nsamp);
  const int v0 = sp * chunk, v1 = min(v0 + chunk, V);
  D2 rr{-INFINITY, -INFINITY, 0x7fffffff}, pp{-INFINITY, -INFINITY, 0x7fffffff};
  int any_r = 0, bad = 0;
  // vector loads need rows of whole 8-id groups on 16-byte boundaries
  const bool vec = (V & 7) == 0 && (reinterpret_cast<uintptr_t>(zt) & 15) == 0 &&
                   (bonus || (reinterpret_cast<uintptr_t>(zd) & 15) == 0);
  constexpr int WIN = 8 * VS_GPT * VS_THREADS;  // ids per window
  // The fp32 bound is formed from the fp32 logit and lse_t rounded to fp32
  // while |lse_t| < 1e30 (then no z / T of the row can overflow fp32, as
  // lse_t >= max z / T), else from the fp64 lp; either way it lies within
  // 2^-21 (|z / T| + |lse_t| + |g| + |bound|) of the exact lp + g.
  const bool f32b = fabs(lse_t) < 1e30;
  const float lse_f = (float)lse_t, invT_f = (float)(1.0 / T);
  // exact values: z / T in fp64; at T = 1 the division is exact and skipped
  // (the walk is instantiated once per case, not chosen per element)
  auto walk = [&](auto unit_c) {
    constexpr bool unit = decltype(unit_c)::value;
    auto over_t = [&](double z) { return unit ? z : z / T; };
    for (int wb = v0; wb < v1; wb += WIN) {
      float uf[VS_GPT][8], gf[VS_GPT][8];
      float ub = -INFINITY;  // this thread's largest bound in the window
#pragma unroll
      for (int gi = 0; gi < VS_GPT; ++gi) {
        const int vb = wb + 8 * (threadIdx.x + gi * VS_THREADS);
        // the 8 target and draft logits are loaded before the noise is drawn,
        // as vectors where the row allows
        float xt[8], xd[8];
        if (vec && vb + 8 <= v1) {
          ld8(zt + vb, xt);
          if (!bonus) ld8(zd + vb, xd);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xt[e] = vb + e < v1 ? ld(zt, vb + e) : 0.f;
            xd[e] = !bonus && vb + e < v1 ? zd[vb + e] : 0.f;
          }
        }
        uint32_t raw[8];
        if (vb < v1)
          philox_block8(a.seed, 2u, (uint64_t)b, (uint64_t)ks, a.cycle, (uint64_t)(vb >> 3), raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = vb + e;
          uf[gi][e] = -INFINITY;
          gf[gi][e] = 0.f;
          if (v >= v1) continue;
          const float g = gumbel_of(raw[e]);
          float bnd;
          if (f32b) bnd = (unit ? xt[e] - lse_f : fmaf(xt[e], invT_f, -lse_f)) + g;
          else bnd = (float)(over_t((double)xt[e]) - lse_t + (double)g);
          uf[gi][e] = bnd;  // -inf where z = -inf; NaN is never a candidate
          gf[gi][e] = g;
          ub = fmaxf(ub, bnd);
          if (!bonus && !isfinite(xd[e])) bad = 1;
        }
      }
      const double U = block_max_d((double)ub, shd);
      if (U == -INFINITY) continue;  // nothing finite in this window
      // covers the fp32 bound's error (above) with a wide margin for every
      // id whose bound is within 16 + |g| of U, and the rounding of tf
      const double slack = 1e-4 + 1e-5 * (fabs(U) + fabs(lse_t));
      // thresholds, highest first; an id is evaluated in the first round
      // whose threshold its bound reaches (done: already evaluated)
      uint32_t done = 0;
#pragma unroll 1
      for (int round = 0; round < 3; ++round) {
        const double t = round == 0 ? U - 4.0 : round == 1 ? U - 16.0 : -INFINITY;
        const float tf = round == 2 ? -INFINITY : (float)(t - slack);
        uint32_t cand = 0;
#pragma unroll
        for (int gi = 0; gi < VS_GPT; ++gi)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (uf[gi][e] > -INFINITY && uf[gi][e] >= tf) cand |= 1u << (8 * gi + e);
        cand &= ~done;
        done |= cand;
        // one fp64 evaluation per candidate, its logits reloaded and its
        // noise taken from the window's registers
        while (cand) {
          const int i = __builtin_ctz(cand);
          cand &= cand - 1;
          const int v = wb + 8 * (threadIdx.x + (i >> 3) * VS_THREADS) + (i & 7);
          float gs = 0.f;
#pragma unroll
          for (int j = 0; j < VS_GPT * 8; ++j) gs = i == j ? gf[j >> 3][j & 7] : gs;
          const double g = (double)gs;
          const double lp = over_t((double)ld(zt, v)) - lse_t;
          d2_push(pp, lp + g, v);
          if (!bonus) {
            const double r = exp(lp) - exp(over_t((double)zd[v]) - lse_d);
            if (r > 0.0) {
              any_r = 1;
              d2_push(rr, log(r) + g, v);
            }
          }
        }
        if (bonus) break;  // the first round decides the bonus draw
        const double best = block_max_d(rr.best, shd);
        if (best >= t + (double)NEAR_BAND + 1e-9) break;
      }
    }
  };
  if (T == 1.0) walk(std::true_type{});
  else walk(std::false_type{});
  for (int o = 32; o > 0; o >>= 1) {
    D2 x{__shfl_xor(rr.best, o, WAVE), __shfl_xor(rr.second, o, WAVE), __shfl_xor(rr.idx, o, WAVE)};
    rr = d2_merge(rr, x);
    D2 y{__shfl_xor(pp.best, o, WAVE), __shfl_xor(pp.second, o, WAVE), __shfl_xor(pp.idx, o, WAVE)};
    pp = d2_merge(pp, y);
    any_r |= __shfl_xor(any_r, o, WAVE);
    bad |= __shfl_xor(bad, o, WAVE);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    VSampPart p;
    p.best_r = rr.best; p.second_r = rr.second; p.idx_r = rr.idx;
    p.best_p = pp.best; p.second_p = pp.second; p.idx_p = pp.idx;
    p.any_r = any_r; p.bad = bad;
    red[wave] = p;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    VSampPart t = red[0];
    for (int i = 1; i < VS_THREADS / 64; ++i) {
      const VSampPart u = red[i];
      D2 x{t.best_r, t.second_r, t.idx_r}, y{u.best_r, u.second_r, u.idx_r};
      x = d2_merge(x, y);
      t.best_r = x.best; t.second_r = x.second; t.idx_r = x.idx;
      D2 xp{t.best_p, t.second_p, t.idx_p}, yp{u.best_p, u.second_p, u.idx_p};
      xp = d2_merge(xp, yp);
      t.best_p = xp.best; t.second_p = xp.second; t.idx_p = xp.idx;
      t.any_r |= u.any_r;
      t.bad |= u.bad;
    }
    w.samp[(long)b * a.nsamp + sp] = t;
  }
}

__global__ __launch_bounds__(64) void vfinish_kernel(VerifyArgs a, VerifyWs w) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int G = a.gamma;
  const int ks = w.kstar[b];
  // lanes over the split records, merged by wave reduction (the top-2 merge
  // with lowest-id ties gives the same result in any order)
  D2 rr{-INFINITY, -INFINITY, 0x7fffffff}, pp{-INFINITY, -INFINITY, 0x7fffffff};
  int any_r = 0, bad = 0;
  for (int sp = lane; sp < a.nsamp; sp += WAVE) {
    const VSampPart p = w.samp[(long)b * a.nsamp + sp];
    rr = d2_merge(rr, D2{p.best_r, p.second_r, p.idx_r});
    pp = d2_merge(pp, D2{p.best_p, p.second_p, p.idx_p});
    any_r |= p.any_r;
    bad |= p.bad;
  }
  for (int o = 32; o > 0; o >>= 1) {
    rr = d2_merge(rr, D2{__shfl_xor(rr.best, o, WAVE), __shfl_xor(rr.second, o, WAVE),
                         __shfl_xor(rr.idx, o, WAVE)});
    pp = d2_merge(pp, D2{__shfl_xor(pp.best, o, WAVE), __shfl_xor(pp.second, o, WAVE),
                         __shfl_xor(pp.idx, o, WAVE)});
    any_r |= __shfl_xor(any_r, o, WAVE);
    bad |= __shfl_xor(bad, o, WAVE);
  }
  if (lane != 0) return;
  uint32_t f = 0;
  int tok;
  double gap;
  if (ks < G && any_r) {
    tok = rr.idx;
    gap = rr.best - rr.second;
  } else {
    if (ks < G) f |= 8u;  // zero residual: drew from p
    tok = pp.idx;
    gap = pp.best - pp.second;
  }
  if (gap < (double)NEAR_BAND) f |= 4u;
  if (bad) f |= 16u;
  a.tokens[(long)b * (G + 1) + ks] = tok;
  a.flags[b] |= f;
}

template <typename TT>
static void launch_typed(const VerifyArgs &a, hipStream_t st) {
  VerifyWs w = carve(a.ws, a.bs, a.gamma, a.nsplit);
  const int rows = a.bs * (a.gamma + 1);
  hipLaunchKernelGGL(vrow_kernel<TT>, dim3(rows, a.nsplit), dim3(256), 0, st, a, w);
  const int dw = a.gamma + 1 < 16 ? a.gamma + 1 : 16;  // one wave per target row, up to 16
  hipLaunchKernelGGL(vdecide_kernel<TT>, dim3(a.bs), dim3(64 * dw), 0, st, a, w);
  if (a.mode == 1) {
    hipLaunchKernelGGL(vsample_kernel<TT>, dim3(a.bs, a.nsamp), dim3(VS_THREADS), 0, st, a, w);
    hipLaunchKernelGGL(vfinish_kernel, dim3(a.bs), dim3(64), 0, st, a, w);
  }
}

void launch_verify(const VerifyArgs &a, hipStream_t st) {
  if (a.bs == 0) return;
  if (a.tdtype == 1) launch_typed<bf16>(a, st);
  else launch_typed<float>(a, st);
}

}  // namespace dstill
