"""Pins for oracle.refine (DStill multi-step refinement).

What fixes it, other than itself:
* the schedule: for every block size and pass count the n_t sum to B - 1
  (every position committed after K passes) and never exceed the masked
  count; K = B - 1 commits one position per pass, K = 1 all at once;
* ranking: brute force with scipy's softmax (max probability) on explicit
  logits, ties to the lower position;
* K = 1 reduces to the one-pass drafter: the endpoint is the greedy head of
  the root state (on the oracle drafter);
* a worked example.
"""

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle.drafter as od
import oracle.refine as rf
from synth import configs, gen

MASK = 49


@pytest.mark.parametrize("B", [2, 5, 16, 33])
def test_schedule_commits_everything(B):
    for K in range(1, B):
        left, total = B - 1, 0
        for t in range(1, K + 1):
            n = rf.n_commit(B, B - left, t, K)
            assert 1 <= n <= left
            left -= n
            total += n
        assert left == 0 and total == B - 1
    # K = B - 1: one per pass; K = 1: all at once
    assert [rf.n_commit(B, 1 + t - 1, t, B - 1) for t in range(1, B)] == [1] * (B - 1)
    assert rf.n_commit(B, 1, 1, 1) == B - 1


def test_ranking_brute_force():
    rng = np.random.default_rng(0)
    B, V = 9, 20
    z = rng.normal(0, 2, (B - 1, V))
    z[4] = z[2]  # a tie between positions 3 and 5
    tokens = np.full(B, MASK)
    tokens[0] = 7
    kappa = np.full(B, -1)
    kappa[0] = 0
    kappa[6], tokens[6] = 1, 3  # already committed
    ids = z.argmax(axis=1)
    t, K = 2, 4
    out, kap = rf.refine_step(tokens, kappa, ids, z.max(axis=1), logsumexp(z, axis=1), t, K)
    conf = softmax(z, axis=1).max(axis=1)
    masked = [i for i in range(1, B) if kappa[i] < 0]
    n = -(-(B - (B - len(masked))) // (K - t + 1))
    order = sorted(masked, key=lambda i: (-round(conf[i - 1], 12), i))[:n]
    assert sorted(np.flatnonzero(kap == t).tolist()) == sorted(order)
    for i in order:
        assert out[i] == ids[i - 1]
    assert out[6] == 3 and kap[6] == 1


def test_worked_example():
    tokens = [5, MASK, MASK, MASK, MASK]
    kappa = [0, -1, -1, -1, -1]
    ids = [10, 11, 12, 13]
    zmax = [1.0, 3.0, 2.0, 3.0]
    lse = [4.0] * 4
    # B = 5, K = 2, t = 1: n = ceil(4 / 2) = 2; slots 2 and 4 tie at -1: both
    out, kap = rf.refine_step(tokens, kappa, ids, zmax, lse, 1, 2)
    assert out.tolist() == [5, MASK, 11, MASK, 13] and kap.tolist() == [0, -1, 1, -1, 1]
    out, kap = rf.refine_step(out, kap, [20, 21, 22, 23], [0.0] * 4, [1.0] * 4, 2, 2)
    assert out.tolist() == [5, 20, 11, 22, 13] and kap.tolist() == [0, 2, 1, 2, 1]


def test_one_pass_is_the_greedy_student():
    base = dict(n_layers=1, hidden=32, n_q_heads=2, n_kv_heads=1, head_dim=16,
                mlp=48, vocab=50, n_feat_layers=2, target_hidden=16, gamma=6,
                dtype="f32", rms_eps=1e-6, rope_theta=1e4, qk_norm=1, bs=1,
                ctx=[7], n_copies=1, verify="greedy", lm_mode="argmax",
                temperature=1.0, target_logit_std=2.0, target_dtype="f32", seed=2)
    cfg = configs.finish(base, "tiny_refine")
    w = gen.weights(cfg)
    npw = {k: (v.float().numpy().astype(np.float64) if not isinstance(v, list)
               else [{a: b.float().numpy().astype(np.float64) for a, b in l.items()} for l in v])
           for k, v in w.items()}
    m = od.Drafter(cfg, npw)
    rng = np.random.default_rng(1)
    S, B = 7, cfg["block"]
    ks, vs = m.inject_rows(rng.normal(0, 1, (S, cfg["feat_dim"])), np.arange(S))
    ck = [k.transpose(1, 0, 2) for k in ks]
    cv = [v.transpose(1, 0, 2) for v in vs]

    def pass_fn(tokens):
        hid = m.draft(ck, cv, [tokens], S)
        h = od.lm_head(npw["lm_head"], hid[0, 1:])
        return h["ids"], h["zmax"], h["lse"]

    x0, kap = rf.rollout(pass_fn, 3, B, 1, cfg["mask_token_id"])
    root = [3] + [cfg["mask_token_id"]] * (B - 1)
    assert x0[1:].tolist() == pass_fn(np.array(root))[0].tolist()
    assert kap.tolist() == [0] + [1] * (B - 1)
    # with more passes every position is committed once, in passes 1..K
    x0, kap = rf.rollout(pass_fn, 3, B, 3, cfg["mask_token_id"])
    assert kap[0] == 0 and set(kap[1:].tolist()) <= {1, 2, 3} and (kap[1:] > 0).all()
