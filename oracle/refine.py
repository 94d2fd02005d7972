"""DStill's multi-step confidence-guided refinement (the teacher rollout), as
a plain definition.  TEST INFRASTRUCTURE ONLY (see the package header).

DStill page, "Multi-step drafting" and the teacher-rollout algorithm of its
appendix ("Training and Trajectory Details"):
* the block starts as x_1 = (anchor, MASK, ..., MASK) with committed set
  c_1 = {0};
* pass t = 1..K runs the drafter on x_t; every masked position i gets the
  confidence conf_i = max_v p_i(v | x_t, H_c);
* n_t = ceil((B - |c_t|) / (K - t + 1)) positions are committed: the n_t
  masked positions of highest confidence, each filled with its greedy
  token; their commit pass is kappa_i = t, earlier commitments stay;
* after K passes every position is committed; x_0 = x_{K+1} is the
  endpoint.

Readings:
  F1  ties in confidence go to the lower position;
  F2  the committed set is tracked by the commit pass (kappa = -1 while
      masked; the anchor has kappa 0), not by comparing tokens with the
      mask id, since a committed greedy token may equal the mask id;
  F3  confidences are ranked as zmax - lse (the log of max_v softmax(z),
      in fp64 from the head's statistics): a monotone image of conf_i;
  F4  the per-pass top-k records of the algorithm (ids and log-probs kept
      for distillation) are training data and are not produced.
"""

from __future__ import annotations

import math

import numpy as np


def n_commit(B, committed, t, K):
    """n_t = ceil((B - |c_t|) / (K - t + 1))."""
    return math.ceil((B - committed) / (K - t + 1))


def refine_step(tokens, kappa, ids, zmax, lse, t, K):
    """One pass.  tokens, kappa [B] (slot 0 the anchor); ids, zmax, lse [B-1]
    the head's outputs for slots 1..B-1 on this pass's state.  Returns the
    updated (tokens, kappa)."""
    tokens = np.array(tokens, copy=True)
    kappa = np.array(kappa, copy=True)
    B = len(tokens)
    masked = [i for i in range(1, B) if kappa[i] < 0]
    n = n_commit(B, B - len(masked), t, K)
    conf = {i: float(np.float64(zmax[i - 1]) - np.float64(lse[i - 1])) for i in masked}
    chosen = sorted(masked, key=lambda i: (-conf[i], i))[:n]
    for i in chosen:
        tokens[i] = int(ids[i - 1])
        kappa[i] = t
    return tokens, kappa


def rollout(pass_fn, anchor, B, K, mask_id):
    """The K-pass rollout; pass_fn(tokens) -> (ids, zmax, lse) for slots
    1..B-1.  Returns the endpoint x_0 and the commit passes kappa."""
    tokens = np.full(B, mask_id, dtype=np.int64)
    tokens[0] = anchor
    kappa = np.full(B, -1, dtype=np.int64)
    kappa[0] = 0
    for t in range(1, K + 1):
        ids, zmax, lse = pass_fn(tokens)
        tokens, kappa = refine_step(tokens, kappa, ids, zmax, lse, t, K)
    return tokens, kappa
