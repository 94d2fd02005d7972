"""Pins for oracle.spot (SPOT state-equality verification).

What fixes the functions, other than themselves:
* commit(): brute force with scipy's softmax: the committed slot is the
  masked slot of largest max-probability at temperature T, its token the
  given id;
* losslessness, the property the page proves: with a deterministic target
  (greedy, or coupled shared-Gumbel noise at T > 0), speculative rounds over
  random draft trees, some of whose drafts follow the target and some not,
  commit exactly the draft-free trajectory;
* a worked example, and the single-path property on trees with duplicate
  drafted states.
"""

import numpy as np
import pytest
from scipy.special import softmax, logsumexp

import oracle.spot as sp

MASK = 99


def _target(V, T, seed):
    """A deterministic synthetic target over block states: per-slot logits
    from a generator seeded by the state's bytes; with T > 0 the committed id
    is the Gumbel-max over a noise table fixed per slot (coupled noise)."""
    noise = np.random.default_rng(seed + 1).gumbel(size=(64, V))

    def f(state):
        rng = np.random.default_rng([seed, abs(hash(tuple(int(t) for t in state))) % (1 << 62)])
        z = rng.normal(0, 2.0, (len(state), V))
        if T == 0:
            ids = z.argmax(axis=1)
            lse = logsumexp(z, axis=1)
            zmax = z.max(axis=1)
        else:
            ids = (z / T + noise[: len(state)]).argmax(axis=1)
            lse = logsumexp(z / T, axis=1)
            zmax = z.max(axis=1)
        return ids, zmax, lse

    return f


def test_commit_brute_force():
    rng = np.random.default_rng(0)
    for T in (1.0, 0.7):
        z = rng.normal(0, 2, (8, 30))
        state = np.array([MASK, 3, MASK, MASK, 7, MASK, MASK, MASK])
        ids = rng.integers(0, 30, 8)
        s, v, _ = sp.commit(state, ids, z.max(axis=1), logsumexp(z / T, axis=1), MASK, T)
        conf = softmax(z / T, axis=1).max(axis=1)
        conf[state != MASK] = -1
        assert s == int(np.argmax(conf)) and v == ids[s]
    # ties: the lowest slot; a full block commits nothing
    assert sp.commit([MASK, MASK], [4, 5], [1.0, 1.0], [2.0, 2.0], MASK)[:2] == (0, 4)
    assert sp.commit([1, 2], [4, 5], [1.0, 1.0], [2.0, 2.0], MASK) is None


def test_worked_example():
    L = 4
    root = np.full(L, MASK)
    ids = np.array([[1, 2, 5, 3], [1, 0, 0, 0], [0, 0, 0, 0], [0, 0, 0, 0]])
    zmax = np.array([[1.0, 1.0, 3.0, 1.0], [2.0, 1.0, 0.0, 1.0], [0.0] * 4, [0.0] * 4])
    lse = np.full((4, L), 4.0)
    states = np.array([root, [MASK, MASK, 5, MASK], [MASK, MASK, 6, MASK], [1, MASK, 5, MASK]])
    parent = [-1, 0, 0, 1]
    commits, deepest, flags = sp.verify_tree(states, parent, ids, zmax, lse, MASK)
    # root commits (2, 5): draft 1 accepted, draft 2 not; draft 1 commits
    # (0, 1): draft 3 accepted; draft 3 then commits at its best slot
    assert deepest == 3
    assert commits[:2] == [(2, 5), (0, 1)]
    assert len(commits) == 3 and flags == sp.FLAG_NEAR_TIE_TARGET  # state 3 has tied slots


@pytest.mark.parametrize("T", [0, 1.0, 1.5])
def test_lossless_against_draft_free(T):
    L, V, D = 8, 12, 6
    tgt = _target(V, T, seed=3)
    rng = np.random.default_rng(5)
    root = np.full(L, MASK)
    Tv = 1.0 if T == 0 else T
    want = sp.decode_draft_free(root, tgt, MASK, Tv)
    assert len(want) == L
    got, x, rounds = [], root.copy(), 0
    while (x == MASK).any():
        # a random tree: each draft extends a random earlier state by one
        # commit, which is the target's own commit with probability 0.6
        states, parent = [x.copy()], [-1]
        for j in range(1, D + 1):
            p = int(rng.integers(0, j))
            ps = states[p]
            m = np.flatnonzero(ps == MASK)
            if m.size == 0:
                states.append(ps.copy()); parent.append(p)
                continue
            if rng.random() < 0.6:
                ids, zmax, lse = tgt(ps)
                s, v, _ = sp.commit(ps, ids, zmax, lse, MASK, Tv)
            else:
                s, v = int(rng.choice(m)), int(rng.integers(0, V))
            states.append(sp.apply(ps, s, v)); parent.append(p)
        outs = [tgt(s_) for s_ in states]
        ids = np.stack([o[0] for o in outs])
        zmax = np.stack([o[1] for o in outs])
        lse = np.stack([o[2] for o in outs])
        commits, deepest, _ = sp.verify_tree(np.stack(states), parent, ids, zmax, lse, MASK,
                                             temperature=Tv)
        for s, v in commits:
            x = sp.apply(x, s, v)
        got += commits
        rounds += 1
    assert got == want
    assert rounds < L  # some drafts were accepted


def test_single_path_with_duplicate_states():
    L = 5
    root = np.full(L, MASK)
    ids = np.tile(np.arange(L), (5, 1))
    zmax = np.tile(np.array([0.0, 0.0, 0.0, 5.0, 0.0]), (5, 1))
    lse = np.full((5, L), 6.0)
    nxt = sp.apply(root, 3, 3)
    states = np.stack([root, nxt, nxt, sp.apply(nxt, 0, 0), sp.apply(nxt, 1, 1)])
    parent = [-1, 0, 0, 2, 1]
    commits, deepest, _ = sp.verify_tree(states, parent, ids, zmax, lse, MASK)
    # drafts 1 and 2 are both the root's next state; the path follows the
    # lower index (draft 1), whose child draft 4 is not its next state; draft
    # 3, accepted under draft 2, is off the path
    assert deepest == 1
    assert commits == [(3, 3), (0, 0)]
