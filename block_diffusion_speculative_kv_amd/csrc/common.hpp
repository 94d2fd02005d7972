// Shared device helpers for the gfx950 kernels: element types, the MFMA
// fragment traits, wave reductions and the Philox4x64-10 generator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace dstill {

// f(std::integral_constant<int, i>{}) for i = 0 .. N - 1, expanded at compile
// time: register arrays indexed by i stay in registers however large the
// body (a plain loop the compiler declines to unroll would index them
// dynamically and move them to scratch memory).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// Near-tie band for every decision flag (same value as DSTILL_NEAR).
constexpr float NEAR_BAND = 1e-5f;

// ---------------------------------------------------------------------------
// MFMA fragment traits.
//
// Every contraction here uses a 16x16 output tile.  A lane l of a wave owns
// the operand fragment of row (l % 16) and "k-group" g = l / 16; each lane
// loads one 16-byte vector, i.e. VEC consecutive k-elements, so one fragment
// covers KW = 4 * VEC values of k.  Because A and B fragments are loaded with
// the same (g, element) -> k mapping, the contraction pairs them correctly
// whatever order the matrix core walks the k slots in.  The 16x16 fp32 result
// lands as: lane l holds D[4 * (l / 16) + i][l % 16], i = 0..3.
//
//   bf16: one v_mfma_f32_16x16x32_bf16 per fragment pair (VEC 8, KW 32)
//   f32 : four v_mfma_f32_16x16x4_f32, element e of every lane in step e
//         (VEC 4, KW 16)
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  typedef bf16x8 frag;
  static constexpr int VEC = 8;
  static constexpr int KW = 32;
  __device__ __forceinline__ static f32x4 run(const frag &a, const frag &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  typedef f32x4 frag;
  static constexpr int VEC = 4;
  static constexpr int KW = 16;
  __device__ __forceinline__ static f32x4 run(const frag &a, const frag &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_frag(const T *p) {
  return *reinterpret_cast<const typename Mma<T>::frag *>(p);
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag zero_frag() {
  typename Mma<T>::frag f;
#pragma unroll
  for (int i = 0; i < Mma<T>::VEC; ++i) f[i] = T(0.0f);
  return f;
}

// ---------------------------------------------------------------------------
// Streaming main loop for weight-bound contractions (few rows): operand
// fragments come straight from global memory into registers, U k-steps at a
// time, into two register banks used in turn, so the loads of the next U
// k-steps are in flight while the current U are multiplied (no register
// copies between banks).  ap[i] / bp[j]: per-lane pointers of the A / B
// operand rows at the first k of the range; nks k-steps of Mma<T>::KW.
// ---------------------------------------------------------------------------
template <typename T, int NA, int NB, int U>
struct StreamBank {
  typename Mma<T>::frag a[U][NA], b[U][NB];
};

template <typename T, int NA, int NB, int U>
__device__ __forceinline__ void stream_load(StreamBank<T, NA, NB, U> &bk, const T *const (&ap)[NA],
                                            const T *const (&bp)[NB], int ks, int nks) {
  constexpr int KW = Mma<T>::KW;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long off = (long)min(ks + u, nks - 1) * KW;  // clamped: in bounds, unused if past nks
#pragma unroll
    for (int i = 0; i < NA; ++i) bk.a[u][i] = load_frag<T>(ap[i] + off);
#pragma unroll
    for (int j = 0; j < NB; ++j) bk.b[u][j] = load_frag<T>(bp[j] + off);
  }
}

template <typename T, int NA, int NB, int U>
__device__ __forceinline__ void stream_mma(const StreamBank<T, NA, NB, U> &bk, int ks, int nks,
                                           f32x4 (&acc)[NA][NB]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (ks + u < nks) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = Mma<T>::run(bk.a[u][i], bk.b[u][j], acc[i][j]);
    }
  }
}

template <typename T, int NA, int NB, int U>
__device__ __forceinline__ void stream_mainloop(const T *const (&ap)[NA], const T *const (&bp)[NB],
                                                int nks, f32x4 (&acc)[NA][NB]) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nks <= 0) return;
  StreamBank<T, NA, NB, U> b0, b1;
  stream_load(b0, ap, bp, 0, nks);
  for (int ks = 0; ks < nks; ks += 2 * U) {
    if (ks + U < nks) stream_load(b1, ap, bp, ks + U, nks);
    stream_mma(b0, ks, nks, acc);
    if (ks + U >= nks) break;
    if (ks + 2 * U < nks) stream_load(b0, ap, bp, ks + 2 * U, nks);
    stream_mma(b1, ks + U, nks, acc);
  }
}

// Groups of k-steps per bank: enough bytes in flight per wave without
// exceeding ~100 fragment registers per bank pair.
template <int NA, int NB>
struct StreamDepth {
  static constexpr int U = (NA + NB) <= 5 ? 4 : ((NA + NB) <= 8 ? 2 : 1);
};

// ---------------------------------------------------------------------------
// Conversions.  float -> bf16 rounds to nearest even (the hardware convert).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024).  `red` is a
// __shared__ scratch of at least blockDim.x / 64 floats.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): per round, two 64x64 -> 128-bit products of
// counter words 0 and 2 with fixed multipliers, a word permutation with the
// key xor-ed into the high halves, then a Weyl bump of the key.
// ---------------------------------------------------------------------------
struct u64x4 { uint64_t w[4]; };

// Full 64 x 64 -> 128-bit product of a constant and x, from four 32 x 32 ->
// 64-bit partial products (each one v_mad_u64_u32): both halves at once.
__device__ __forceinline__ void mulhilo64(uint64_t m, uint64_t x, uint64_t &lo, uint64_t &hi) {
  const uint64_t ml = (uint32_t)m, mh = m >> 32, xl = (uint32_t)x, xh = x >> 32;
  const uint64_t p0 = ml * xl;                    // bits 0..63
  const uint64_t p1 = ml * xh + (p0 >> 32);       // bits 32..95, cannot overflow
  const uint64_t p2 = mh * xl + (uint32_t)p1;     // bits 32..95, cannot overflow
  lo = (p2 << 32) | (uint32_t)p0;
  hi = mh * xh + (p1 >> 32) + (p2 >> 32);
}

__device__ __forceinline__ u64x4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                               uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t lo0, hi0, lo1, hi1;
    mulhilo64(M0, c0, lo0, hi0);
    mulhilo64(M1, c2, lo1, hi1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0; k1 += W1;
  }
  u64x4 o; o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
  return o;
}

// Stream layout: counter = (j / 8, pos, seq, cycle << 8 | purpose), key =
// (seed, 0); element j is 32-bit half (j % 2, high half first) of 64-bit word
// (j / 2) % 4.  One call yields elements 8t .. 8t+7.
__device__ __forceinline__ void philox_block8(uint64_t seed, uint32_t purpose, uint64_t seq,
                                              uint64_t pos, uint64_t cycle, uint64_t t,
                                              uint32_t out[8]) {
  const u64x4 r = philox4x64_10(t, pos, seq, (cycle << 8) | purpose, seed, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (uint32_t)(r.w[i] >> 32);
    out[2 * i + 1] = (uint32_t)(r.w[i] & 0xffffffffu);
  }
}

// u = ((x >> 8) | 1) * 2^-24: odd multiples of 2^-24 in [2^-24, 1 - 2^-24],
// exact in fp32.
__device__ __forceinline__ float u24(uint32_t x) {
  return (float)((x >> 8) | 1u) * 5.9604644775390625e-08f;
}

// Standard Gumbel draw g = -log(-log u), through the hardware base-2
// logarithm (v_log_f32, ~1 ulp on the normal inputs that occur here: u and
// -log u lie in [2^-25, 17.4]); g is off by a few ulp, far inside the
// near-tie band that decides which argmaxes are compared exactly.
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  constexpr float LN2 = 0.6931471805599453f;
  return -LN2 * __builtin_amdgcn_logf(-LN2 * __builtin_amdgcn_logf(u24(x)));
}

// Argmax merge with lowest-index tie-break; `second` tracks the runner-up
// score (for the near-tie band).
struct ArgTop2 {
  float best, second;
  int idx;
};
// Selects rather than branches: the update runs once per logit in the
// vocabulary sweeps, where divergent branches cost more than both sides.
__device__ __forceinline__ void top2_push(ArgTop2 &a, float s, int i) {
  const bool win = s > a.best || (s == a.best && i < a.idx);
  a.second = fmaxf(a.second, win ? a.best : s);
  a.best = win ? s : a.best;
  a.idx = win ? i : a.idx;
}
// top2_push for a chain that sees its ids in increasing order and finite
// values only: a later id wins only when strictly greater, so the runner-up
// is max(second, min(best, s)).
__device__ __forceinline__ void top2_push_inc(ArgTop2 &a, float s, int i) {
  a.idx = s > a.best ? i : a.idx;
  a.second = fmaxf(a.second, fminf(a.best, s));
  a.best = fmaxf(a.best, s);
}
__device__ __forceinline__ ArgTop2 top2_merge(ArgTop2 a, ArgTop2 b) {
  if (b.best > a.best || (b.best == a.best && b.idx < a.idx)) {
    ArgTop2 t = a; a = b; b = t;
  }
  a.second = fmaxf(a.second, b.best);
  return a;
}

__device__ __forceinline__ ArgTop2 top2_shfl_xor(ArgTop2 a, int o) {
  ArgTop2 b;
  b.best = __shfl_xor(a.best, o, WAVE);
  b.second = __shfl_xor(a.second, o, WAVE);
  b.idx = __shfl_xor(a.idx, o, WAVE);
  return top2_merge(a, b);
}

}  // namespace dstill
