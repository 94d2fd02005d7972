// Per-row and element-wise stages of the drafter, each fused onto the output
// of a projection: summing the k-split partial planes, RMSNorm with its gain,
// per-head q/k RMSNorm with the rotary embedding, the SwiGLU gate, and the
// scatter of injected K/V into the cache.
//
// Readings of the drafter (DStill appendix drafter table: "Qwen3-style"
// layers; DFlash review, Method / Inference for the injection):
//   RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g, in fp32;
//   rotary embedding on q and k: the pair (i, i + dh/2) turns by the angle
//   pos * theta^(-2i/dh), computed in fp64 so that positions up to 2^20 keep
//   full fp32 accuracy;
//   SwiGLU: silu(gate) * up, silu(x) = x / (1 + exp(-x)).
// Layouts: K is stored as dh-vectors ([cap][dh] per sequence and kv head),
// V in tiles of 64 keys, d-major inside a tile ([cap/64][dh][64]; block V in
// the workspace as [dh][16]): the layout the attention kernel's P.V operand
// reads as contiguous blocks.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dstill {

// ---- context clamp, token check ----------------------------------------------
__global__ __launch_bounds__(64) void draft_prep_kernel(const int32_t *__restrict__ tokens,
                                                        const int32_t *__restrict__ ctx_len,
                                                        int per_seq, int vocab, int ctx_limit,
                                                        int32_t *__restrict__ eff_ctx,
                                                        int32_t *__restrict__ tok_clamped,
                                                        uint32_t *__restrict__ flags) {
  const int b = blockIdx.x, lane = threadIdx.x;
  uint32_t f = 0;
  for (int i = lane; i < per_seq; i += WAVE) {
    int t = tokens[(long)b * per_seq + i];
    if (t < 0 || t >= vocab) {
      f |= 16u;  // DSTILL_FLAG_BAD_INPUT
      t = t < 0 ? 0 : vocab - 1;
    }
    tok_clamped[(long)b * per_seq + i] = t;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, WAVE);
  if (lane == 0) {
    int c = ctx_len[b];
    if (c < 0 || c > ctx_limit) {
      f |= 32u;  // DSTILL_FLAG_CTX_CLAMPED
      c = c < 0 ? 0 : ctx_limit;
    }
    eff_ctx[b] = c;
    if (flags) flags[b] = f;
  }
}

void launch_draft_prep(const int32_t *tokens, const int32_t *ctx_len, int bs, int per_seq,
                       int vocab, int ctx_limit, int32_t *eff_ctx, int32_t *tok_clamped,
                       uint32_t *flags, hipStream_t st) {
  hipLaunchKernelGGL(draft_prep_kernel, dim3(bs), dim3(64), 0, st, tokens, ctx_len, per_seq, vocab,
                     ctx_limit, eff_ctx, tok_clamped, flags);
}

// ---- embedding gather into the fp32 residual stream --------------------------
// One workgroup per row.  Rows whose width is a multiple of 8 move as
// 8-element vectors, the loads of a thread issued before its stores, so a
// row costs about one round trip to memory instead of one per element.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T *__restrict__ embed,
                                                    const int32_t *__restrict__ tok, int d,
                                                    float *__restrict__ h) {
  const int r = blockIdx.x;
  const T *src = embed + (long)tok[r] * d;
  float *dst = h + (long)r * d;
  if (d % 8 == 0) {
    constexpr int U = 4;  // vectors in flight per thread
    for (int j0 = 8 * threadIdx.x; j0 < d; j0 += 8 * U * blockDim.x) {
      float x[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + 8 * u * blockDim.x;
        if (j < d) {
          if constexpr (sizeof(T) == 2) {
            const bf16x8 v = *reinterpret_cast<const bf16x8 *>(src + j);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[u][e] = static_cast<float>(v[e]);
          } else {
            const f32x4 v0 = *reinterpret_cast<const f32x4 *>(src + j);
            const f32x4 v1 = *reinterpret_cast<const f32x4 *>(src + j + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[u][e] = v0[e];
              x[u][4 + e] = v1[e];
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + 8 * u * blockDim.x;
        if (j < d) {
          *reinterpret_cast<f32x4 *>(dst + j) = f32x4{x[u][0], x[u][1], x[u][2], x[u][3]};
          *reinterpret_cast<f32x4 *>(dst + j + 4) = f32x4{x[u][4], x[u][5], x[u][6], x[u][7]};
        }
      }
    }
  } else {
    for (int j = threadIdx.x; j < d; j += blockDim.x) dst[j] = to_f32(src[j]);
  }
}

void launch_embed(int dtype, const void *embed, const int32_t *tok, int R, int d, float *h,
                  hipStream_t st) {
  if (R == 0) return;
  if (dtype == 1)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(R), dim3(256), 0, st, (const bf16 *)embed, tok, d, h);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(R), dim3(256), 0, st, (const float *)embed, tok, d, h);
}

// ---- RMSNorm over rows, fused with the split-sum and the residual add --------
// Two passes, each over a grid of (row, 1024-column chunk) workgroups so that
// even a handful of rows keeps the GPU busy: (1) x = resid + sum of the
// partial planes (fixed order), written back as the new residual (or to a
// scratch row), with the chunk's sum of squares; (2) out = x * rs * gain with
// rs = 1 / sqrt(mean(x^2) + eps) from the chunk sums (fixed order).
constexpr int NORM_CHUNK = 1024;  // columns per workgroup (256 threads x 4)

__global__ __launch_bounds__(256) void split_sum_kernel(const float *__restrict__ parts,
                                                        int nsplit, int M, int d,
                                                        const float *resid, float *xout,
                                                        float *__restrict__ ssp, int nchunk) {
  __shared__ float red[4];
  const int r = blockIdx.x, ch = blockIdx.y;
  const int c = ch * NORM_CHUNK + threadIdx.x * 4;
  float ss = 0.f;
  if (c < d) {
    f32x4 x = resid ? *reinterpret_cast<const f32x4 *>(resid + (long)r * d + c)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < nsplit; ++sp)
      x += *reinterpret_cast<const f32x4 *>(parts + ((long)sp * M + r) * d + c);
    if (xout) *reinterpret_cast<f32x4 *>(xout + (long)r * d + c) = x;
    ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  }
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) ssp[(long)r * nchunk + ch] = ss;
}

template <typename T>
__global__ __launch_bounds__(256) void norm_apply_kernel(const float *__restrict__ x, int d,
                                                         const float *__restrict__ ssp, int nchunk,
                                                         const T *__restrict__ gain, float eps,
                                                         T *__restrict__ out, long out_stride) {
  const int r = blockIdx.x, ch = blockIdx.y;
  float ss = 0.f;
  for (int i = 0; i < nchunk; ++i) ss += ssp[(long)r * nchunk + i];
  const float rs = 1.0f / sqrtf(ss / (float)d + eps);
  const int c = ch * NORM_CHUNK + threadIdx.x * 4;
  if (c >= d) return;
  const f32x4 v = *reinterpret_cast<const f32x4 *>(x + (long)r * d + c);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    out[(long)r * out_stride + c + e] = from_f32<T>(v[e] * rs * to_f32(gain[c + e]));
}

// One workgroup per row, the whole row in registers (d <= 4096 CPT): the
// split-sum, the residual write-back, the sum of squares and the scaled
// output in a single pass, with no scratch row.  Partial planes are summed in
// split order, as in the two-pass form.
constexpr int NORM_ROW_T = 1024;
template <typename T, int CPT, int NT = NORM_ROW_T>
__global__ __launch_bounds__(NT) void norm_row_kernel(
    const float *__restrict__ parts, int nsplit, int M, int d, float *resid, int write_resid,
    const T *__restrict__ gain, float eps, T *__restrict__ out, long out_stride) {
  __shared__ float red[NT / WAVE];
  const int r = blockIdx.x;
  f32x4 x[CPT];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = (i * NT + threadIdx.x) * 4;
    x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c < d) {
      if (resid) x[i] = *reinterpret_cast<const f32x4 *>(resid + (long)r * d + c);
      // the planes in batches of SB loads in flight, summed in split order
      constexpr int SB = 8;
      for (int sp0 = 0; sp0 < nsplit; sp0 += SB) {
        f32x4 pv[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k)
          if (sp0 + k < nsplit)
            pv[k] = *reinterpret_cast<const f32x4 *>(parts + ((long)(sp0 + k) * M + r) * d + c);
#pragma unroll
        for (int k = 0; k < SB; ++k)
          if (sp0 + k < nsplit) x[i] += pv[k];
      }
      if (resid && write_resid) *reinterpret_cast<f32x4 *>(resid + (long)r * d + c) = x[i];
      ss += x[i][0] * x[i][0] + x[i][1] * x[i][1] + x[i][2] * x[i][2] + x[i][3] * x[i][3];
    }
  }
  ss = block_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = (i * NT + threadIdx.x) * 4;
    if (c >= d) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      out[(long)r * out_stride + c + e] = from_f32<T>(x[i][e] * rs * to_f32(gain[c + e]));
  }
}

template <typename T>
static bool launch_norm_row(const float *parts, int nsplit, int M, int d, float *resid,
                            int write_resid, const void *gain, float eps, void *out,
                            long out_stride, hipStream_t st) {
  const int cpt = (d + 4 * NORM_ROW_T - 1) / (4 * NORM_ROW_T);
  auto go = [&](auto kern, int nt) {
    hipLaunchKernelGGL(kern, dim3(M), dim3(nt), 0, st, parts, nsplit, M, d, resid, write_resid,
                       (const T *)gain, eps, (T *)out, out_stride);
  };
  // many rows (prefill chunks): 256 threads with 4x the columns each, so a
  // compute unit keeps 4x the bytes in flight
  if (M >= 2048 && d <= 4096) {
    go(norm_row_kernel<T, 4, 256>, 256);
    return true;
  }
  if (cpt == 1) go(norm_row_kernel<T, 1>, NORM_ROW_T);
  else if (cpt == 2) go(norm_row_kernel<T, 2>, NORM_ROW_T);
  else if (cpt <= 4) go(norm_row_kernel<T, 4>, NORM_ROW_T);
  else return false;
  return true;
}

void launch_norm_rows(int dtype, const float *parts, int nsplit, int M, int d, float *resid,
                      int write_resid, const void *gain, float eps, void *out, long out_stride,
                      float *xtmp, float *ssp, hipStream_t st) {
  if (M == 0) return;
  if (d % 4 == 0) {
    const bool done = dtype == 1 ? launch_norm_row<bf16>(parts, nsplit, M, d, resid, write_resid,
                                                         gain, eps, out, out_stride, st)
                                 : launch_norm_row<float>(parts, nsplit, M, d, resid, write_resid,
                                                          gain, eps, out, out_stride, st);
    if (done) return;
  }
  const int nchunk = (d + NORM_CHUNK - 1) / NORM_CHUNK;
  // where x lives for the second pass
  float *xout = (resid && write_resid) ? resid : ((nsplit > 0 || !resid) ? xtmp : nullptr);
  const float *xsrc = xout ? xout : resid;
  dim3 grid(M, nchunk);
  hipLaunchKernelGGL(split_sum_kernel, grid, dim3(256), 0, st, parts, nsplit, M, d,
                     (const float *)resid, xout, ssp, nchunk);
  if (dtype == 1)
    hipLaunchKernelGGL(norm_apply_kernel<bf16>, grid, dim3(256), 0, st, xsrc, d, ssp, nchunk,
                       (const bf16 *)gain, eps, (bf16 *)out, out_stride);
  else
    hipLaunchKernelGGL(norm_apply_kernel<float>, grid, dim3(256), 0, st, xsrc, d, ssp, nchunk,
                       (const float *)gain, eps, (float *)out, out_stride);
}

// ---- rotary table: (cos, sin) of every rotary pair of every row ------------
// angle = pos * theta^(-2p/dh), in fp64, rounded to fp32 once; every head of
// a row reads the same row of the table.
__global__ __launch_bounds__(64) void rope_table_kernel(const int32_t *__restrict__ eff_ctx,
                                                        int rows_per_seq, int block,
                                                        const int32_t *__restrict__ pos, int dh,
                                                        float theta, float2 *__restrict__ tab) {
  const int r = blockIdx.x, half = dh / 2;
  const int p = blockIdx.y * 64 + threadIdx.x;
  if (p >= half) return;
  const int ps = pos ? max(pos[r], 0) : eff_ctx[r / rows_per_seq] + r % block;
  const double inv = exp(-2.0 * (double)p / (double)dh * log((double)theta));
  double sn, cs;
  sincos((double)ps * inv, &sn, &cs);
  tab[(long)r * half + p] = make_float2((float)cs, (float)sn);
}

void launch_rope_table(const int32_t *eff_ctx, int rows_per_seq, int block, const int32_t *pos,
                       int n, int dh, float theta, float *tab, hipStream_t st) {
  if (n == 0) return;
  hipLaunchKernelGGL(rope_table_kernel, dim3(n, (dh / 2 + 63) / 64), dim3(64), 0, st, eff_ctx,
                     rows_per_seq, block, pos, dh, theta, (float2 *)tab);
}

// ---- per-head RMSNorm + rotary embedding -------------------------------------
// One wave handles one (row, head); lane p owns the rotary pairs
// (p, p + dh/2) and (p + 64, p + 64 + dh/2) (dh <= 256); cs is the row's
// rotary table.
__device__ __forceinline__ void rope_pair(float &x1, float &x2, float2 cs) {
  const float y1 = x1 * cs.x - x2 * cs.y;
  const float y2 = x2 * cs.x + x1 * cs.y;
  x1 = y1;
  x2 = y2;
}

// The same with the gains and the rotary table already in registers (g1[i],
// g2[i], c[i] for p = lane + 64 i), so a caller can request them ahead.
__device__ __forceinline__ void head_norm_rope_regs(float x1[2], float x2[2], int dh, bool norm,
                                                    const float g1[2], const float g2[2],
                                                    float eps, const float2 c[2]) {
  const int lane = threadIdx.x & 63, half = dh / 2;
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) ss += x1[i] * x1[i] + x2[i] * x2[i];
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)dh + eps);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = lane + 64 * i;
      if (p < half) {
        x1[i] = x1[i] * rs * g1[i];
        x2[i] = x2[i] * rs * g2[i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = lane + 64 * i;
    if (p < half) rope_pair(x1[i], x2[i], c[i]);
  }
}

template <typename T>
__device__ __forceinline__ void head_norm_rope(float x1[2], float x2[2], int dh, bool norm,
                                               const T *g, float eps,
                                               const float2 *__restrict__ cs) {
  const int lane = threadIdx.x & 63, half = dh / 2;
  float g1[2] = {0.f, 0.f}, g2[2] = {0.f, 0.f};
  float2 c[2] = {float2{1.f, 0.f}, float2{1.f, 0.f}};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = lane + 64 * i;
    if (p < half) {
      if (norm) {
        g1[i] = to_f32(g[p]);
        g2[i] = to_f32(g[p + half]);
      }
      c[i] = cs[p];
    }
  }
  head_norm_rope_regs(x1, x2, dh, norm, g1, g2, eps, c);
}

// Wide head layout for 128-dim heads: 16 lanes per (row, head), lane l
// holding dims 4l .. 4l + 3 (a) and 64 + 4l .. 64 + 4l + 3 (c), so each
// rotary pair (e, e + 64) sits in one lane.  Optional RMSNorm over the 128
// dims (a reduction over the 16 lanes) with gains g1 / g2, then the rotary
// embedding with the row's (cos, sin) of dims 4l .. 4l + 3 (c01, c23).
__device__ __forceinline__ void wide_norm_rope(float a[4], float c[4], bool norm, const float g1[4],
                                               const float g2[4], float eps, f32x4 c01,
                                               f32x4 c23) {
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += a[e] * a[e] + c[e] * c[e];
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, WAVE);
    const float rs = 1.0f / sqrtf(ss / 128.0f + eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = a[e] * rs * g1[e];
      c[e] = c[e] * rs * g2[e];
    }
  }
  const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) rope_pair(a[e], c[e], float2{cs[2 * e], cs[2 * e + 1]});
}

constexpr int POST_HEADS = 4;  // heads per workgroup, one wave each
// Rows per workgroup of the injection's head pass: per-row work is small, so
// with many rows each wave takes its head in a few consecutive rows (fewer,
// longer waves); with few rows one, so the launch still fills the chip.  (The
// same change left the drafter's per-layer head pass at bs 32 unchanged.)
static int post_rows(int n) { return n >= 256 ? 4 : 1; }
template <typename T>
__global__ __launch_bounds__(64 * POST_HEADS) void qkv_post_kernel(
    const float *__restrict__ parts, int nsplit, int R, int hq, int hkv, int dh,
    const int32_t *__restrict__ eff_ctx, int rows_per_seq, int block,
    const T *__restrict__ q_norm, const T *__restrict__ k_norm, int qk_norm, float eps,
    const float2 *__restrict__ rope, T *__restrict__ q, T *__restrict__ kb, T *__restrict__ vb) {
  const int r = blockIdx.x, head = blockIdx.y * POST_HEADS + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = dh / 2, ncol = (hq + 2 * hkv) * dh;
  if (head >= hq + 2 * hkv) return;
  const bool is_q = head < hq, is_k = !is_q && head < hq + hkv;
  float x1[2] = {0.f, 0.f}, x2[2] = {0.f, 0.f};
  // the planes in batches of SB loads in flight, summed in split order
  constexpr int SB = 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = lane + 64 * i;
    if (p < half) {
      const float *src = parts + (long)r * ncol + head * dh + p;
      for (int s0 = 0; s0 < nsplit; s0 += SB) {
        float a1[SB], a2[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k)
          if (s0 + k < nsplit) {
            a1[k] = src[(long)(s0 + k) * R * ncol];
            a2[k] = src[(long)(s0 + k) * R * ncol + half];
          }
#pragma unroll
        for (int k = 0; k < SB; ++k)
          if (s0 + k < nsplit) {
            x1[i] += a1[k];
            x2[i] += a2[k];
          }
      }
    }
  }
  if (!is_q && !is_k) {
    // block V, d-major per (sequence-copy, kv head): [dh][16 key slots]
    T *dst = vb + (((long)(r / block) * hkv + (head - hq - hkv)) * dh) * 16 + r % block;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = lane + 64 * i;
      if (p < half) {
        dst[(long)p * 16] = from_f32<T>(x1[i]);
        dst[(long)(p + half) * 16] = from_f32<T>(x2[i]);
      }
    }
    return;
  }
  T *dst = is_q ? q + (long)r * hq * dh + head * dh : kb + (long)r * hkv * dh + (head - hq) * dh;
  head_norm_rope<T>(x1, x2, dh, qk_norm != 0, is_q ? q_norm : k_norm, eps, rope + (long)r * half);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = lane + 64 * i;
    if (p < half) {
      dst[p] = from_f32<T>(x1[i]);
      dst[p + half] = from_f32<T>(x2[i]);
    }
  }
}

void launch_qkv_post(int dtype, const float *parts, int nsplit, int R, int hq, int hkv, int dh,
                     const int32_t *eff_ctx, int rows_per_seq, int block, const void *q_norm,
                     const void *k_norm, int qk_norm, float eps, const float *rope, void *q,
                     void *kb, void *vb, hipStream_t st) {
  if (R == 0) return;
  dim3 grid(R, (hq + 2 * hkv + POST_HEADS - 1) / POST_HEADS);
  if (dtype == 1)
    hipLaunchKernelGGL(qkv_post_kernel<bf16>, grid, dim3(64 * POST_HEADS), 0, st, parts, nsplit, R, hq, hkv, dh,
                       eff_ctx, rows_per_seq, block, (const bf16 *)q_norm, (const bf16 *)k_norm,
                       qk_norm, eps, (const float2 *)rope, (bf16 *)q, (bf16 *)kb, (bf16 *)vb);
  else
    hipLaunchKernelGGL(qkv_post_kernel<float>, grid, dim3(64 * POST_HEADS), 0, st, parts, nsplit, R, hq, hkv, dh,
                       eff_ctx, rows_per_seq, block, (const float *)q_norm, (const float *)k_norm,
                       qk_norm, eps, (const float2 *)rope, (float *)q, (float *)kb, (float *)vb);
}

// ---- SwiGLU gate ------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const float *__restrict__ parts, int nsplit,
                                                     int R, int mlp, T *__restrict__ act) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)R * mlp) return;
  const long r = i / mlp, j = i % mlp;
  const long plane = (long)R * 2 * mlp;
  float g = 0.f, u = 0.f;
  // the planes in batches of SB loads in flight, summed in split order
  constexpr int SB = 8;
  for (int s0 = 0; s0 < nsplit; s0 += SB) {
    float gv[SB], uv[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k)
      if (s0 + k < nsplit) {
        gv[k] = parts[(s0 + k) * plane + r * 2 * mlp + j];
        uv[k] = parts[(s0 + k) * plane + r * 2 * mlp + mlp + j];
      }
#pragma unroll
    for (int k = 0; k < SB; ++k)
      if (s0 + k < nsplit) {
        g += gv[k];
        u += uv[k];
      }
  }
  const float silu = g / (1.0f + expf(-g));
  act[i] = from_f32<T>(silu * u);
}

void launch_swiglu(int dtype, const float *parts, int nsplit, int R, int mlp, void *act,
                   hipStream_t st) {
  const long n = (long)R * mlp;
  if (n == 0) return;
  const int blocks = (int)((n + 255) / 256);
  if (dtype == 1)
    hipLaunchKernelGGL(swiglu_kernel<bf16>, dim3(blocks), dim3(256), 0, st, parts, nsplit, R, mlp,
                       (bf16 *)act);
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3(blocks), dim3(256), 0, st, parts, nsplit, R, mlp,
                       (float *)act);
}

// ---- injected K/V: k-norm + rotary embedding, scatter into the cache --------
template <typename T, int RPW>
__global__ __launch_bounds__(64 * POST_HEADS) void inject_post_kernel(
    const float *__restrict__ parts, int nsplit, int n, int hkv, int dh,
    const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, InjectLayers il,
    int qk_norm, float eps, const float2 *__restrict__ rope, int max_batch, int cap,
    int with_v) {
  // K heads, and the V heads too when with_v (else inject_v_kernel does them);
  // each wave takes its head in RPW consecutive rows, whose split-plane
  // loads are all issued before the first row is normalised and stored
  const int head = blockIdx.y * POST_HEADS + (threadIdx.x >> 6);
  const int layer = blockIdx.z, lane = threadIdx.x & 63;
  if (head >= (with_v ? 2 : 1) * hkv) return;
  const int half = dh / 2, ncol = 2 * hkv * dh, width = il.layers * ncol;
  const bool is_k = head < hkv;
  const int h = is_k ? head : head - hkv;
  T *kc = (T *)il.kc[layer], *vc = (T *)il.vc[layer];
  float x1[RPW][2], x2[RPW][2];
  int sq[RPW], ps[RPW];
  // the rows' ids, rotary tables and (K) the norm gains are requested
  // together with the planes
  const bool norm = is_k && qk_norm != 0;
  float g1[2] = {0.f, 0.f}, g2[2] = {0.f, 0.f};
  float2 cs[RPW][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = lane + 64 * j;
    if (norm && p < half) {
      g1[j] = to_f32(((const T *)il.k_norm[layer])[p]);
      g2[j] = to_f32(((const T *)il.k_norm[layer])[p + half]);
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = blockIdx.x * RPW + i;
    sq[i] = r < n ? seq[r] : -1;
    ps[i] = r < n ? pos[r] : -1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      x1[i][j] = x2[i][j] = 0.f;
      const int p = lane + 64 * j;
      cs[i][j] = is_k && r < n && p < half ? rope[(long)r * half + p] : float2{1.f, 0.f};
    }
  }
  // splits outermost, so every load of one split is in flight at once (sums
  // in split order)
  for (int s = 0; s < nsplit; ++s) {
    const float *plane = parts + (long)s * n * width + layer * ncol + head * dh;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = blockIdx.x * RPW + i;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int p = lane + 64 * j;
        if (r < n && p < half) {
          x1[i][j] += plane[(long)r * width + p];
          x2[i][j] += plane[(long)r * width + p + half];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = blockIdx.x * RPW + i;
    if (r >= n) break;
    if (sq[i] < 0 || sq[i] >= max_batch || ps[i] < 0 || ps[i] >= cap) continue;
    // K cache rows are dh-vectors [cap][dh]; the V cache is stored in tiles
    // of 64 keys, d-major inside a tile: [cap/64][dh][64]
    const long stride = is_k ? 1 : 64;
    T *dst = is_k ? kc + (((long)sq[i] * hkv + h) * cap + ps[i]) * dh
                  : vc + ((long)sq[i] * hkv + h) * dh * cap + (long)(ps[i] >> 6) * dh * 64 +
                        (ps[i] & 63);
    if (is_k) head_norm_rope_regs(x1[i], x2[i], dh, norm, g1, g2, eps, cs[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = lane + 64 * j;
      if (p < half) {
        dst[p * stride] = from_f32<T>(x1[i][j]);
        dst[(p + half) * stride] = from_f32<T>(x2[i][j]);
      }
    }
  }
}

// K heads of many rows with dh = 128 (bf16): 16 lanes per (row, head), each
// lane holding 4 consecutive dims of each half (the rotary pairs (e, e + 64)
// in one lane), so loads are 16 bytes and a wave has 4 rows of its head in
// flight per batch, KW_BATCH batches issued before any is finished.  The
// head norm reduces over the 16 lanes of a row.
constexpr int KW_BATCH = 2;
constexpr int KW_ROWS = 4 * 4 * KW_BATCH;  // rows per workgroup (4 waves)
template <typename T>
__global__ __launch_bounds__(256) void inject_k_wide_kernel(
    const float *__restrict__ parts, int nsplit, int n, int hkv, const int32_t *__restrict__ seq,
    const int32_t *__restrict__ pos, InjectLayers il, int qk_norm, float eps,
    const float2 *__restrict__ rope, int max_batch, int cap) {
  constexpr int DH = 128, HALF = 64;
  const int h = blockIdx.y, layer = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = lane >> 4, l = lane & 15;
  const int ncol = 2 * hkv * DH, width = il.layers * ncol;
  const bool norm = qk_norm != 0;
  float g1[4], g2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    g1[e] = norm ? to_f32(((const T *)il.k_norm[layer])[4 * l + e]) : 1.f;
    g2[e] = norm ? to_f32(((const T *)il.k_norm[layer])[HALF + 4 * l + e]) : 1.f;
  }
  f32x4 x1[KW_BATCH], x2[KW_BATCH], c01[KW_BATCH], c23[KW_BATCH];
  int rr[KW_BATCH], sq[KW_BATCH], ps[KW_BATCH];
#pragma unroll
  for (int b = 0; b < KW_BATCH; ++b) {
    const int r = blockIdx.x * KW_ROWS + wave * 4 * KW_BATCH + 4 * b + sub;
    rr[b] = r;
    sq[b] = r < n ? seq[r] : -1;
    ps[b] = r < n ? pos[r] : -1;
    x1[b] = x2[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the row's rotary table: (cos, sin) of dims 4l .. 4l + 3
    const f32x4 *cr = reinterpret_cast<const f32x4 *>(rope + (long)min(r, n - 1) * HALF + 4 * l);
    c01[b] = cr[0];
    c23[b] = cr[1];
  }
  for (int s = 0; s < nsplit; ++s) {
    const float *plane = parts + (long)s * n * width + layer * ncol + h * DH + 4 * l;
#pragma unroll
    for (int b = 0; b < KW_BATCH; ++b) {
      if (rr[b] < n) {
        x1[b] += *reinterpret_cast<const f32x4 *>(plane + (long)rr[b] * width);
        x2[b] += *reinterpret_cast<const f32x4 *>(plane + (long)rr[b] * width + HALF);
      }
    }
  }
  T *kc = (T *)il.kc[layer];
#pragma unroll
  for (int b = 0; b < KW_BATCH; ++b) {
    float a[4], c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = x1[b][e];
      c[e] = x2[b][e];
    }
    wide_norm_rope(a, c, norm, g1, g2, eps, c01[b], c23[b]);
    T o1[4], o2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o1[e] = from_f32<T>(a[e]);
      o2[e] = from_f32<T>(c[e]);
    }
    if (rr[b] >= n || sq[b] < 0 || sq[b] >= max_batch || ps[b] < 0 || ps[b] >= cap) continue;
    T *dst = kc + (((long)sq[b] * hkv + h) * cap + ps[b]) * DH + 4 * l;
    *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(o1);
    *reinterpret_cast<uint2 *>(dst + HALF) = *reinterpret_cast<const uint2 *>(o2);
  }
}

// V rows of the injected layers, 64 rows x dh per workgroup: the split sums
// are staged in LDS as [row][d] (loads along d) and written out along rows,
// so the rows of consecutive positions of one sequence, which share a 64-key
// tile of the d-major V cache, fill consecutive 2-byte slots of each tile
// row.  Sums in split order, one rounding to the cache dtype, as for K.
constexpr int INJ_VROWS = 64;
constexpr int INJ_V_MIN_ROWS = 2048;
template <typename T>
__global__ __launch_bounds__(256) void inject_v_kernel(
    const float *__restrict__ parts, int nsplit, int n, int hkv, int dh,
    const int32_t *__restrict__ seq, const int32_t *__restrict__ pos, InjectLayers il,
    int max_batch, int cap) {
  extern __shared__ float tile[];  // [INJ_VROWS][dh + 1]
  __shared__ int rsq[INJ_VROWS], rps[INJ_VROWS], gsq[INJ_VROWS / 8], gps[INJ_VROWS / 8];
  const int r0 = blockIdx.x * INJ_VROWS, h = blockIdx.y, layer = blockIdx.z;
  // the rows' sequence ids and positions are requested first and staged in
  // LDS with the tile
  int my_sq = -1, my_ps = -1;
  if (threadIdx.x < INJ_VROWS && r0 + (int)threadIdx.x < n) {
    my_sq = seq[r0 + threadIdx.x];
    my_ps = pos[r0 + threadIdx.x];
  }
  const int ncol = 2 * hkv * dh, width = il.layers * ncol, ts = dh + 1;
  const long col0 = (long)layer * ncol + (long)hkv * dh + (long)h * dh;
  // 16-byte loads, eight per thread issued together (dh is 64 or 128)
  const int q4 = dh / 4;
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < INJ_VROWS * q4; i0 += U * blockDim.x) {
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // splits outermost: the U loads of a split are in flight together
    for (int s = 0; s < nsplit; ++s) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * blockDim.x, row = i / q4, r = r0 + row;
        if (i < INJ_VROWS * q4 && r < n)
          x[u] += *reinterpret_cast<const f32x4 *>(parts + (long)s * n * width + (long)r * width +
                                                   col0 + 4 * (i % q4));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * blockDim.x;
      if (i >= INJ_VROWS * q4) break;
      const int row = i / q4, d = 4 * (i % q4);
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[row * ts + d + e] = x[u][e];
    }
  }
  // groups of 8 rows that are 8 consecutive positions of one sequence from a
  // multiple of 8 (the usual prefill case) fill 8 consecutive slots of a tile
  // row: one 16-byte store; other groups are stored element by element
  if (threadIdx.x < INJ_VROWS) {
    rsq[threadIdx.x] = my_sq;
    rps[threadIdx.x] = my_ps;
  }
  __syncthreads();
  if (threadIdx.x < INJ_VROWS / 8) {
    const int g = 8 * threadIdx.x;
    int q = rsq[g];
    const int p0 = rps[g];
    bool ok = r0 + g + 7 < n && q >= 0 && q < max_batch && p0 >= 0 && p0 + 7 < cap &&
              (p0 & 7) == 0;
#pragma unroll
    for (int e = 1; e < 8; ++e) ok = ok && rsq[g + e] == q && rps[g + e] == p0 + e;
    gsq[threadIdx.x] = ok ? q : -1;
    gps[threadIdx.x] = p0;
  }
  __syncthreads();
  T *vc = (T *)il.vc[layer];
  for (int i = threadIdx.x; i < (INJ_VROWS / 8) * dh; i += blockDim.x) {
    const int d = i / (INJ_VROWS / 8), grp = i % (INJ_VROWS / 8), row0 = 8 * grp;
    const int q = gsq[grp];
    if (q >= 0) {
      const int p0 = gps[grp];
      T v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(tile[(row0 + e) * ts + d]);
      T *dst = vc + ((long)q * hkv + h) * dh * cap + (long)(p0 >> 6) * dh * 64 + (long)d * 64 +
               (p0 & 63);
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = v[e];
      }
      continue;
    }
    for (int e = 0; e < 8; ++e) {
      const int row = row0 + e, r = r0 + row;
      if (r >= n) break;
      const int sq = rsq[row], ps = rps[row];
      if (sq < 0 || sq >= max_batch || ps < 0 || ps >= cap) continue;
      vc[((long)sq * hkv + h) * dh * cap + (long)(ps >> 6) * dh * 64 + (long)d * 64 + (ps & 63)] =
          from_f32<T>(tile[row * ts + d]);
    }
  }
}

// The per-row head pass: K heads (norm + rotary), and V heads when with_v.
template <typename T>
static void launch_post_rows(const float *parts, int nsplit, int n, int hkv, int dh,
                             const int32_t *seq, const int32_t *pos, const InjectLayers &il,
                             int qk_norm, float eps, const float *rope, int max_batch, int cap,
                             int with_v, hipStream_t st) {
  const int rpw = post_rows(n);
  const dim3 grid((n + rpw - 1) / rpw, ((with_v ? 2 : 1) * hkv + POST_HEADS - 1) / POST_HEADS,
                  il.layers);
  const float2 *cs = (const float2 *)rope;
  if (rpw == 4)
    hipLaunchKernelGGL((inject_post_kernel<T, 4>), grid, dim3(64 * POST_HEADS), 0, st, parts,
                       nsplit, n, hkv, dh, seq, pos, il, qk_norm, eps, cs, max_batch, cap, with_v);
  else
    hipLaunchKernelGGL((inject_post_kernel<T, 1>), grid, dim3(64 * POST_HEADS), 0, st, parts,
                       nsplit, n, hkv, dh, seq, pos, il, qk_norm, eps, cs, max_batch, cap, with_v);
}

void launch_inject_post(int dtype, const float *parts, int nsplit, int n, int hkv, int dh,
                        const int32_t *seq, const int32_t *pos, const InjectLayers &il,
                        int qk_norm, float eps, const float *rope, int max_batch, int cap,
                        hipStream_t st) {
  if (n == 0 || il.layers == 0) return;
  // K heads: per-head norm + rotary embedding, one wave per (row, head), or
  // (bf16, dh 128, from INJ_V_MIN_ROWS rows) the wide pass with 16 lanes per
  // (row, head).  V heads: with few rows the same per-row pass (enough
  // workgroups), from INJ_V_MIN_ROWS rows the row-tiled transposing pass
  // (contiguous stores).
  const int with_v = n < INJ_V_MIN_ROWS;
  if (dtype == 1 && !with_v && dh == 128) {
    const dim3 kgrid((n + KW_ROWS - 1) / KW_ROWS, hkv, il.layers);
    hipLaunchKernelGGL(inject_k_wide_kernel<bf16>, kgrid, dim3(256), 0, st, parts, nsplit, n, hkv,
                       seq, pos, il, qk_norm, eps, (const float2 *)rope, max_batch, cap);
  } else if (dtype == 1) {
    launch_post_rows<bf16>(parts, nsplit, n, hkv, dh, seq, pos, il, qk_norm, eps, rope, max_batch,
                           cap, with_v, st);
  } else {
    launch_post_rows<float>(parts, nsplit, n, hkv, dh, seq, pos, il, qk_norm, eps, rope,
                            max_batch, cap, with_v, st);
  }
  if (with_v) return;
  // V heads: staged and written along rows
  const dim3 vgrid((n + INJ_VROWS - 1) / INJ_VROWS, hkv, il.layers);
  const size_t lds = (size_t)INJ_VROWS * (dh + 1) * sizeof(float);
  if (dtype == 1)
    hipLaunchKernelGGL(inject_v_kernel<bf16>, vgrid, dim3(256), lds, st, parts, nsplit, n, hkv, dh,
                       seq, pos, il, max_batch, cap);
  else
    hipLaunchKernelGGL(inject_v_kernel<float>, vgrid, dim3(256), lds, st, parts, nsplit, n, hkv,
                       dh, seq, pos, il, max_batch, cap);
}

}  // namespace dstill
