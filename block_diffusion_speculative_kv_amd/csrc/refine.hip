// One pass of DStill's multi-step confidence-guided refinement (DStill page,
// "Multi-step drafting" and the teacher rollout of its appendix): after the
// drafter and the LM head have scored the current block state, the n_t =
// ceil((B - |c_t|) / (K - t + 1)) masked positions of highest confidence
// take their greedy tokens and record commit pass t; earlier commitments
// stay.  The drafter pass and the head are the ordinary library calls on the
// current block tokens; this kernel only updates the state between passes.
//
// One wave per sequence, lane i = block slot i (B <= 64).  Masked slots are
// those with commit pass < 0 (a committed token may equal the mask id).  The
// confidence max_v softmax(z) is ranked through zmax - lse in fp64; lane i
// is committed iff fewer than n_t masked slots rank above it (larger
// confidence, or equal confidence at a lower slot).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dstill {

__global__ __launch_bounds__(64) void refine_commit_kernel(RefineArgs a) {
  const int b = blockIdx.x, i = threadIdx.x;
  const int B = a.block;
  const long row = (long)b * B;
  const bool masked = i >= 1 && i < B && a.kappa[row + i] < 0;
  const long hr = (long)b * (B - 1) + (i - 1);  // head row of slot i
  const double conf = masked ? (double)a.zmax[hr] - (double)a.lse[hr] : -INFINITY;
  const int n_masked = __popcll(__ballot(masked));
  const int committed = B - n_masked;
  const int left = a.K - a.t + 1;
  const int n = left > 0 ? (B - committed + left - 1) / left : 0;
  int rank = 0;
  for (int j = 1; j < B; ++j) {
    const double cj = __shfl(conf, j, WAVE);
    const bool mj = __shfl((int)masked, j, WAVE) != 0;
    if (mj && (cj > conf || (cj == conf && j < i))) ++rank;
  }
  if (masked && rank < n) {
    a.tokens[row + i] = a.ids[hr];
    a.kappa[row + i] = a.t;
  }
}

void launch_refine_commit(const RefineArgs &a, hipStream_t st) {
  if (a.bs == 0) return;
  hipLaunchKernelGGL(refine_commit_kernel, dim3(a.bs), dim3(64), 0, st, a);
}

}  // namespace dstill
