// SPOT state-equality verification over a draft tree (SPOT page, section 4:
// the target commits at the masked slot of highest confidence, writing the
// token drawn with noise shared per slot, so its commit is a deterministic
// function of the state; a drafted state is accepted iff it equals its
// parent's next state and the parent is accepted, so the accepted drafts
// form one path; the round emits the commits along that path and the commit
// of its deepest state).
//
// Inputs are the per-slot head outputs of every state (root = state 0, then
// the drafts), as the multi-copy layout produces them: ids (the
// shared-Gumbel argmax), zmax and lse at temperature T, and the winner's gap.
// One wave per sequence, lanes over the slots of a state (L <= 64) and over
// the states (n <= 64); the tree's states and slot confidences are staged in
// LDS first by one pass of independent loads:
//   1. per state: confidence zmax/T - lse in fp64 over its masked slots, the
//      wave's top-2 (ties to the lowest slot) -> committed slot, token and
//      the near-tie bits;
//   2. per draft, in index order (a parent precedes its children): state
//      equality with the parent's next state, by ballot over the slots;
//   3. the path from the root, each step to the lowest accepted child.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dstill {

constexpr double SPOT_NEAR = 1e-5;  // compared in fp64, as the decision values are

__global__ __launch_bounds__(64) void spot_verify_kernel(SpotArgs a) {
  __shared__ int sstar[64], vstar[64];
  __shared__ uint32_t nflag[64];
  __shared__ int acc[64];
  __shared__ int st[64 * 64];       // states, [n][L]
  __shared__ double cf[64 * 64];    // confidences of masked slots, -inf elsewhere
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = a.n_states, L = a.L;
  const long base = (long)b * n * L;
  const double T = (double)a.temperature;
  // every state and confidence of the tree in one pass of independent loads
  for (int k = lane; k < n * L; k += WAVE) {
    const int t = a.states[base + k];
    st[k] = t;
    cf[k] = t == a.mask_id ? (double)a.zmax[base + k] / T - (double)a.lse[base + k] : -INFINITY;
  }
  __syncthreads();
  for (int i = 0; i < n; ++i) {
    const bool masked = lane < L && st[i * L + lane] == a.mask_id;
    double best = masked ? cf[i * L + lane] : -INFINITY;
    double second = -INFINITY;
    int bi = masked ? lane : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o, WAVE), os = __shfl_xor(second, o, WAVE);
      const int oi = __shfl_xor(bi, o, WAVE);
      const bool take = ob > best || (ob == best && oi < bi);
      second = fmax(fmax(second, os), take ? best : ob);
      best = take ? ob : best;
      bi = take ? oi : bi;
    }
    if (lane == 0) {
      const bool any = bi != 0x7fffffff;
      sstar[i] = any ? bi : -1;
      vstar[i] = any ? a.ids[base + (long)i * L + bi] : -1;
      uint32_t f = 0;
      if (any && best - second < SPOT_NEAR) f |= 1u;  // near-tie slot choice
      if (any && a.gap && (double)a.gap[base + (long)i * L + bi] < SPOT_NEAR) f |= 4u;
      nflag[i] = f;
    }
  }
  __syncthreads();
  if (lane == 0) acc[0] = 1;
  __syncthreads();
  for (int j = 1; j < n; ++j) {
    const int p = a.parent[(long)b * n + j];
    const bool ok = p >= 0 && p < j && acc[p] && sstar[p] >= 0;  // wave-uniform
    bool eq = true;
    if (ok && lane < L) {
      const int want = lane == sstar[p] ? vstar[p] : st[p * L + lane];
      eq = st[j * L + lane] == want;
    }
    const bool all = __ballot(!eq) == 0;
    if (lane == 0) acc[j] = ok && all;
    __syncthreads();
  }
  // the accepted path from the root
  int cur = 0, cnt = 0;
  uint32_t flags = 0;
  const long ob = (long)b * n;
  for (;;) {
    const int j = lane;
    const bool child = j > 0 && j < n && acc[j] && a.parent[ob + j] == cur;
    const unsigned long long m = __ballot(child);
    flags |= nflag[cur];
    if (sstar[cur] >= 0) {
      if (lane == 0) {
        a.out_slots[ob + cnt] = sstar[cur];
        a.out_tokens[ob + cnt] = vstar[cur];
      }
      ++cnt;
    }
    if (!m) break;
    cur = __builtin_ctzll(m);
  }
  for (int k = cnt + lane; k < n; k += WAVE) {
    a.out_slots[ob + k] = -1;
    a.out_tokens[ob + k] = -1;
  }
  if (lane == 0) {
    a.out_n[b] = cnt;
    a.out_state[b] = cur;
    a.out_flags[b] = flags;
  }
}

void launch_spot_verify(const SpotArgs &a, hipStream_t st) {
  if (a.bs == 0) return;
  hipLaunchKernelGGL(spot_verify_kernel, dim3(a.bs), dim3(64), 0, st, a);
}

}  // namespace dstill
