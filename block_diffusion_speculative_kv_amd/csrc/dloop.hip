// D-Loop's looped second draft pass and its joint K-branch verification
// (D-Loop page, section 3.1: prefix score, top-K prefix lengths, remasked
// suffix re-drafted by the same drafter, Eq. (4)-(5); section 3.3: one target
// pass over all branches, the longest matching prefix is committed).
//
// The drafter itself is not repeated here: the K branch blocks are drafted
// as K copies of the block behind the shared context (the multi-copy layout
// of the draft kernels), and their slots 1..m go through the LM head as
// usual.  This file adds the three small steps around that pass:
//   dloop_branch_kernel  confidences c_k = exp(zmax_k - lse_k) (fp64), the
//                        prefix scores r_l = (c_1..c_l)(1 - c_{l+1}) taken
//                        left to right, the K best lengths (ties to the
//                        smaller l) and each branch's block tokens;
//   dloop_merge_kernel   branch proposal = first-pass prefix + second-pass
//                        suffix;
//   branch_pick_kernel   after a greedy verification of every branch: the
//                        branch with the largest tau (ties to the lowest
//                        index), its tokens, and the OR of every branch's
//                        flags (a near tie in any branch can change which is
//                        longest).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dstill {

// One wave per sequence; m = gamma <= 63, K <= m.
__global__ __launch_bounds__(64) void dloop_branch_kernel(DloopArgs a) {
  __shared__ double r[64];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int m = a.gamma;
  if (lane == 0) {
    // left to right, as the definition reads: r_l = P_l (1 - c_{l+1})
    double prod = 1.0;
    for (int l = 0; l < m; ++l) {
      const double c = exp((double)a.zmax[(long)b * m + l] - (double)a.lse[(long)b * m + l]);
      r[l] = prod * (1.0 - c);
      prod *= c;
    }
  }
  __syncthreads();
  // K rounds of an argmax over the lanes (lane l holds r_l), each round
  // taking the largest remaining score, the smaller l on ties
  const bool mine = lane < m;
  double v = mine ? r[lane] : 0.0;
  bool taken = !mine;
  int lens_lane = 0;  // lane j < K ends up with branch j's length
  for (int j = 0; j < a.K; ++j) {
    double bv = taken ? -1.0 : v;  // scores are >= 0
    int bl = taken ? 0x7fffffff : lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o, WAVE);
      const int ol = __shfl_xor(bl, o, WAVE);
      if (ov > bv || (ov == bv && ol < bl)) {
        bv = ov;
        bl = ol;
      }
    }
    if (lane == bl) taken = true;
    if (lane == j) lens_lane = bl;
    if (lane == 0) {
      a.prefix_len[(long)b * a.K + j] = bl;
      if (a.score) a.score[(long)b * a.K + j] = bv;
    }
  }
  // block tokens: branch j, slot s (lanes over slots, m + 1 <= 64)
  for (int j = 0; j < a.K; ++j) {
    const int l = __shfl(lens_lane, j, WAVE);
    if (lane <= m) {
      int t = a.mask_id;
      if (lane == 0) t = a.anchor[b];
      else if (lane <= l) t = a.ids[(long)b * m + lane - 1];
      a.block_tokens[((long)b * a.K + j) * (m + 1) + lane] = t;
    }
  }
}

__global__ __launch_bounds__(64) void dloop_merge_kernel(int gamma, int K,
                                                         const int32_t *__restrict__ first,
                                                         const int32_t *__restrict__ second,
                                                         const int32_t *__restrict__ lens,
                                                         int32_t *__restrict__ out) {
  const int b = blockIdx.x, j = blockIdx.y, k = threadIdx.x;
  if (k >= gamma) return;
  const long br = (long)b * K + j;
  out[br * gamma + k] = k < lens[br] ? first[(long)b * gamma + k] : second[br * gamma + k];
}

__global__ __launch_bounds__(64) void branch_pick_kernel(int K, int gamma,
                                                         const int32_t *__restrict__ tok,
                                                         const int32_t *__restrict__ tau,
                                                         const uint32_t *__restrict__ flags,
                                                         int32_t *__restrict__ out_tokens,
                                                         int32_t *__restrict__ out_tau,
                                                         int32_t *__restrict__ out_branch,
                                                         uint32_t *__restrict__ out_flags) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int best = 0, bt = -1;
  uint32_t f = 0;
  for (int j = 0; j < K; ++j) {
    const int t = tau[(long)b * K + j];
    f |= flags[(long)b * K + j];
    if (t > bt) {
      bt = t;
      best = j;
    }
  }
  if (lane <= gamma)
    out_tokens[(long)b * (gamma + 1) + lane] = tok[((long)b * K + best) * (gamma + 1) + lane];
  if (lane == 0) {
    out_tau[b] = bt;
    if (out_branch) out_branch[b] = best;
    out_flags[b] = f;
  }
}

void launch_dloop_branches(const DloopArgs &a, hipStream_t st) {
  if (a.bs == 0) return;
  hipLaunchKernelGGL(dloop_branch_kernel, dim3(a.bs), dim3(64), 0, st, a);
}

void launch_dloop_merge(int bs, int gamma, int K, const int32_t *first, const int32_t *second,
                        const int32_t *lens, int32_t *out, hipStream_t st) {
  if (bs == 0) return;
  hipLaunchKernelGGL(dloop_merge_kernel, dim3(bs, K), dim3(64), 0, st, gamma, K, first, second,
                     lens, out);
}

void launch_branch_pick(int bs, int K, int gamma, const int32_t *tok, const int32_t *tau,
                        const uint32_t *flags, int32_t *out_tokens, int32_t *out_tau,
                        int32_t *out_branch, uint32_t *out_flags, hipStream_t st) {
  if (bs == 0) return;
  hipLaunchKernelGGL(branch_pick_kernel, dim3(bs), dim3(64), 0, st, K, gamma, tok, tau, flags,
                     out_tokens, out_tau, out_branch, out_flags);
}

}  // namespace dstill
