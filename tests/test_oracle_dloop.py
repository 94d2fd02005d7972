"""Pins for oracle.dloop (D-Loop second pass, joint K-branch verification).

What fixes each function, other than itself:
* prefix scores: the telescoping identity sum_l r_l + prod_k c_k = 1 (each
  r_l is the chance that independent acceptances with probabilities c_k
  first fail at position l + 1), checked against a Monte Carlo of exactly
  that process, and a worked example computed by hand;
* confidences: scipy's softmax probability of the argmax token;
* selection: brute force over all orderings on small m, with planted ties;
* branch blocks and merge: worked examples;
* two-pass wiring: a branch with l = 0 is the first-pass block, so its
  second-pass tokens equal the first-pass proposal; with l = m nothing is
  re-drafted;
* joint verification: planted matches give every tau, the longest branch
  wins, ties go to the lowest branch.
"""

import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle.dloop as dl
import oracle.drafter as od
from synth import configs, gen


def test_prefix_scores_worked_example():
    # c = (0.9, 0.5, 0.8): r0 = 0.1, r1 = 0.9 * 0.5, r2 = 0.9 * 0.5 * 0.2
    r = dl.prefix_scores([0.9, 0.5, 0.8])
    assert np.allclose(r, [0.1, 0.45, 0.09], rtol=0, atol=1e-15)
    assert dl.select_lengths(r, 1) == [1]
    assert dl.select_lengths(r, 3) == [1, 0, 2]


def test_prefix_scores_telescope_and_first_failure_law():
    rng = np.random.default_rng(0)
    for m in (1, 3, 7, 15):
        c = rng.uniform(0.05, 0.999, m)
        r = dl.prefix_scores(c)
        assert np.all(r >= 0)
        assert abs(r.sum() + np.prod(c) - 1.0) < 1e-14
    # Monte Carlo of the first failure position of independent Bernoulli(c_k)
    c = np.array([0.8, 0.6, 0.9, 0.3, 0.7])
    acc = rng.random((400_000, c.size)) < c
    first = np.where(acc.all(axis=1), c.size, np.argmin(acc, axis=1))
    freq = np.bincount(first, minlength=c.size + 1)[: c.size] / acc.shape[0]
    assert np.allclose(freq, dl.prefix_scores(c), atol=3e-3)


def test_confidence_is_softmax_of_argmax():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 3, (6, 40))
    zmax = z.max(axis=1)
    lse = np.log(np.exp(z).sum(axis=1))
    c = dl.confidences(zmax, lse)
    assert np.allclose(c, softmax(z, axis=1).max(axis=1), rtol=1e-13)


def test_selection_matches_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for _ in range(50):
        m = int(rng.integers(1, 6))
        r = np.round(rng.uniform(0, 1, m), 1)  # coarse values: ties are common
        for K in range(1, m + 1):
            got = dl.select_lengths(r, K)
            # brute force: the lexicographically smallest (by -r, then l)
            # sequence among all K-permutations that are sorted by -r
            best = None
            for perm in itertools.permutations(range(m), K):
                keyseq = [(-r[l], l) for l in perm]
                if keyseq != sorted(keyseq):
                    continue
                rest = [l for l in range(m) if l not in perm]
                if rest and max(r[l] for l in rest) > min(r[l] for l in perm):
                    continue
                if best is None or keyseq < [(-r[l], l) for l in best]:
                    best = perm
            assert got == list(best)
    # a planted exact tie: c = (0.5, 0.0) gives r0 = r1 = 0.5
    r = dl.prefix_scores([0.5, 0.0])
    assert r[0] == r[1] == 0.5
    assert dl.select_lengths(r, 2) == [0, 1]


def test_branch_blocks_and_merge():
    ids = [11, 12, 13, 14]
    blocks = dl.branch_blocks(7, ids, [2, 0, 4], mask_id=99)
    assert blocks.tolist() == [[7, 11, 12, 99, 99], [7, 99, 99, 99, 99], [7, 11, 12, 13, 14]]
    second = [[21, 22, 23, 24], [31, 32, 33, 34], [41, 42, 43, 44]]
    out = dl.merge(ids, second, [2, 0, 4])
    assert out.tolist() == [[11, 12, 23, 24], [31, 32, 33, 34], [11, 12, 13, 14]]


def _tiny():
    base = dict(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                mlp=96, vocab=50, n_feat_layers=3, target_hidden=32, gamma=5,
                dtype="f32", rms_eps=1e-6, rope_theta=1e4, qk_norm=1, bs=1,
                ctx=[9], n_copies=3, verify="greedy", lm_mode="argmax",
                temperature=1.0, target_logit_std=2.0, target_dtype="f32",
                seed=5)
    return configs.finish(base, "tiny_dloop")


def test_two_pass_wiring_on_the_oracle_drafter():
    cfg = _tiny()
    w = gen.weights(cfg)
    npw = {k: (v.float().numpy().astype(np.float64) if not isinstance(v, list)
               else [{a: b.float().numpy().astype(np.float64) for a, b in l.items()} for l in v])
           for k, v in w.items()}
    m = od.Drafter(cfg, npw)
    rng = np.random.default_rng(3)
    S, g, mask = 9, cfg["gamma"], cfg["vocab"] - 1
    ks, vs = m.inject_rows(rng.normal(0, 1, (S, cfg["feat_dim"])), np.arange(S))
    ck = [k.transpose(1, 0, 2) for k in ks]
    cv = [v.transpose(1, 0, 2) for v in vs]
    anchor = 4
    first = m.draft(ck, cv, [[anchor] + [mask] * g], S)
    h1 = od.lm_head(npw["lm_head"], first[0, 1:])
    blocks, lens, _ = dl.dloop_branches(anchor, h1["ids"], h1["zmax"], h1["lse"], 3, mask)
    # force the l = 0 and l = m branches in as well
    blocks = np.concatenate([blocks, dl.branch_blocks(anchor, h1["ids"], [0, g], mask)])
    lens = list(lens) + [0, g]
    second = m.draft(ck, cv, blocks, S)
    ids2 = np.stack([od.lm_head(npw["lm_head"], second[j, 1:])["ids"] for j in range(len(lens))])
    final = dl.merge(h1["ids"], ids2, lens)
    # l = 0: the branch block is the first-pass block, so it drafts the same tokens
    assert np.array_equal(ids2[-2], h1["ids"])
    assert np.array_equal(final[-2], h1["ids"])
    # l = m: the proposal is the first pass unchanged
    assert np.array_equal(final[-1], h1["ids"])
    # every branch keeps its prefix
    for j, l in enumerate(lens):
        assert np.array_equal(final[j][:l], h1["ids"][:l])


def test_joint_verification_planted():
    rng = np.random.default_rng(4)
    K, g, V = 4, 6, 30
    y = rng.integers(0, V, (K, g))
    zt = rng.normal(0, 1, (K, g + 1, V))
    planted = [2, 5, 5, 1]  # accepted prefix per branch
    for k in range(K):
        for j in range(g + 1):
            zt[k, j, :] -= 10.0 * (np.arange(V) == (y[k, j] if j < g else 0))
        for j in range(planted[k]):
            zt[k, j, y[k, j]] += 20.0
    toks, tau, br, flags = dl.verify_branches_greedy(zt, y)
    assert tau == 6 and br == 1  # branches 1 and 2 tie at L = 5: the lower wins
    assert toks[:5] == [int(t) for t in y[1, :5]]
    assert toks[5] == int(np.argmax(zt[1, 5]))
    assert flags == 0
    # single branch reduces to the one-sequence rule
    t1, tau1, br1, f1 = dl.verify_branches_greedy(zt[:1], y[:1])
    assert (tau1, br1) == (3, 0)
