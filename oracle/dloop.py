"""D-Loop's looped second draft pass and joint K-branch greedy verification,
as plain definitions.  TEST INFRASTRUCTURE ONLY (see the package header).

D-Loop page, section 3.1 ("From one-pass marginals to a prefix-conditioned
loop", Eq. (4)-(5) and the prefix score that follows them):

* the first pass drafts the whole block from z0 = (anchor, MASK x m) and
  proposes x~_1..x~_m with confidences c_k = q_k(x~_k | C, z0);
* each prefix length l in 0..m-1 is scored by
  r_l = (c_1 * ... * c_l) * (1 - c_{l+1});
* the K best lengths are kept; for each, the block (anchor, x~_1..x~_l,
  MASK, ..., MASK) is drafted again by the same drafter, and the branch's
  proposal is x~_1..x~_l followed by the second pass's tokens l+1..m.

D-Loop page, section 3.3 (inference and verification): with K > 1 branches
one target pass scores every branch; the longest matching prefix is
committed together with the target's correction or bonus token.

Readings where the page leaves a step open:
  D1  c_k is the first-pass softmax probability of the proposed token at
      temperature 1; with greedy drafting the proposal is the argmax, so
      c_k = exp(zmax_k - lse_k), from the LM head's per-row statistics.
  D2  ties in r_l go to the smaller l; branches are listed by decreasing r.
  D3  the committed branch is the one with the largest tau (accepted prefix
      + 1); ties go to the lowest branch index.
  D4  each branch has its own target rows (the branch-specific causal
      attention makes the target's logits differ per branch); its greedy
      verification is the one-sequence rule, and the flags of every branch
      are OR-ed, since a near tie in any branch can change which is longest.

Layouts: ids, zmax, lse [bs, m] (first pass, slots 1..m); branch blocks
[bs, K, m + 1]; second-pass ids [bs, K, m]; target logits [bs, K, m + 1, V].
"""

from __future__ import annotations

import numpy as np

from .verify import verify_greedy


def confidences(zmax, lse):
    """c_k = exp(zmax_k - lse_k) in fp64 (reading D1)."""
    return np.exp(np.asarray(zmax, dtype=np.float64) - np.asarray(lse, dtype=np.float64))


def prefix_scores(c):
    """r_l = (prod_{k <= l} c_k)(1 - c_{l+1}) for l = 0..m-1 (c[k-1] is c_k)."""
    c = np.asarray(c, dtype=np.float64)
    m = c.shape[-1]
    r = np.empty(m, dtype=np.float64)
    prod = 1.0
    for l in range(m):
        r[l] = prod * (1.0 - c[l])
        prod *= c[l]
    return r


def select_lengths(r, K):
    """The K best prefix lengths by r, decreasing, ties to the smaller l (D2)."""
    order = sorted(range(len(r)), key=lambda l: (-float(r[l]), l))
    return order[:K]


def branch_blocks(anchor, ids, lengths, mask_id):
    """Block tokens of every branch: (anchor, x~_1..x~_l, MASK...), m + 1 slots."""
    m = len(ids)
    out = []
    for l in lengths:
        out.append([int(anchor)] + [int(t) for t in ids[:l]] + [int(mask_id)] * (m - l))
    return np.asarray(out, dtype=np.int64)


def merge(ids, second, lengths):
    """Branch proposals: x~_1..x~_l then the second pass's tokens l+1..m."""
    m = len(ids)
    out = []
    for j, l in enumerate(lengths):
        out.append([int(ids[k]) if k < l else int(second[j][k]) for k in range(m)])
    return np.asarray(out, dtype=np.int64)


def dloop_branches(anchor, ids, zmax, lse, K, mask_id):
    """One sequence: (block tokens [K, m+1], lengths [K], scores [K])."""
    r = prefix_scores(confidences(zmax, lse))
    lens = select_lengths(r, K)
    return branch_blocks(anchor, ids, lens, mask_id), np.asarray(lens), r[lens]


def verify_branches_greedy(zt, y):
    """zt [K, m+1, V] target logits of each branch, y [K, m] branch proposals.
    Returns (tokens, tau, branch, flags) of the committed branch (D3, D4)."""
    best = None
    flags = 0
    for k in range(len(y)):
        toks, tau, f = verify_greedy(zt[k], y[k])
        flags |= f
        if best is None or tau > best[1]:
            best = (toks, tau, k)
    return best[0], best[1], best[2], flags
