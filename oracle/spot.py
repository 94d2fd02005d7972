"""SPOT state-equality verification over a draft tree, as a plain definition.
TEST INFRASTRUCTURE ONLY (see the package header).

SPOT page, section 4 (problem setting and verification):
* a block state x holds a token or the mask symbol at each of its L slots;
  one target forward gives, for every masked slot s, the conditional
  p_s(. | x, C);
* the target commits at s*(x) = the masked slot with the highest
  confidence max_v p_s(v | x, C), writing the argmax token at T = 0 or, at
  T > 0, a token drawn from the temperature-adjusted conditional; with
  coupled noise the draw is the Gumbel-max over a noise table shared per
  slot, so the commit is again a deterministic function of the state;
* D drafted states, each with a parent in a tree rooted at the current
  state, are scored in the same forward as the root; a draft is accepted
  iff it equals its parent's next state x_parent + (s*, v*) (state
  equality) and its parent is accepted.  The commits are unique, so the
  accepted drafts form one path; the round emits the commits along it and
  the commit of its deepest state (that state was scored too).

Readings:
  S1  the confidence of a masked slot is the head's tempered statistic
      max_v softmax(z_s / T) = exp(zmax_s / T - lse_s); at T = 1 (the
      multi-copy workload) it is the page's max_v p_s;
  S2  ties in confidence go to the lowest slot; the committed token is the
      head's shared-Gumbel argmax id of that slot;
  S3  a state with no masked slot commits nothing; a draft whose parent
      index is not an earlier state is never accepted; when several
      accepted children of one state exist (equal drafted states), the
      path follows the lowest index;
  S4  near ties are flagged, not resolved: FLAG_NEAR_TIE_TARGET when a
      state on the emitted path has its two best confidences within 1e-5,
      FLAG_NEAR_TIE_SAMPLE when a commit on it has a head gap below 1e-5.
"""

from __future__ import annotations

import numpy as np

NEAR = 1e-5
FLAG_NEAR_TIE_TARGET = 1
FLAG_NEAR_TIE_SAMPLE = 4


def commit(state, ids, zmax, lse, mask_id, temperature=1.0):
    """Next commit of one state: (slot, token, confidence gap) or None."""
    state = np.asarray(state)
    masked = np.flatnonzero(state == mask_id)
    if masked.size == 0:
        return None
    conf = np.asarray(zmax, np.float64)[masked] / float(temperature) - \
        np.asarray(lse, np.float64)[masked]
    k = int(np.argmax(conf))  # first maximum: the lowest slot on ties
    rest = np.delete(conf, k)
    gap = conf[k] - (rest.max() if rest.size else -np.inf)
    s = int(masked[k])
    return s, int(ids[s]), gap


def apply(state, s, v):
    out = np.array(state, copy=True)
    out[s] = v
    return out


def verify_tree(states, parent, ids, zmax, lse, mask_id, temperature=1.0, gap=None):
    """states [n, L] (state 0 = root), parent [n] (parent[0] ignored),
    ids / zmax / lse / gap [n, L]: the target's per-slot head outputs for
    every state.  Returns (commits [(slot, token)], deepest accepted state,
    flags)."""
    n = len(states)
    com = [commit(states[i], ids[i], zmax[i], lse[i], mask_id, temperature) for i in range(n)]
    acc = [False] * n
    acc[0] = True
    for j in range(1, n):
        p = int(parent[j])
        if 0 <= p < j and acc[p] and com[p] is not None:
            s, v, _ = com[p]
            acc[j] = bool(np.array_equal(states[j], apply(states[p], s, v)))
    path = [0]
    while True:
        kids = [j for j in range(1, n) if acc[j] and int(parent[j]) == path[-1]]
        if not kids:
            break
        path.append(kids[0])
    commits, flags = [], 0
    for i in path:
        if com[i] is None:
            continue
        s, v, g = com[i]
        if g < NEAR:
            flags |= FLAG_NEAR_TIE_TARGET
        if gap is not None and gap[i][s] < NEAR:
            flags |= FLAG_NEAR_TIE_SAMPLE
        commits.append((s, v))
    return commits, path[-1], flags


def decode_draft_free(state, target, mask_id, temperature=1.0, max_steps=None):
    """Draft-free decoding: one commit per target forward until the block is
    full.  target(state) -> (ids, zmax, lse) per slot."""
    x = np.array(state, copy=True)
    traj = []
    steps = 0
    while (x == mask_id).any() and (max_steps is None or steps < max_steps):
        ids, zmax, lse = target(x)
        s, v, _ = commit(x, ids, zmax, lse, mask_id, temperature)
        x = apply(x, s, v)
        traj.append((s, v))
        steps += 1
    return traj
