"""Pins for the oracle's verification and sampling steps.

* Losslessness of rejection-sampling verification, by exact enumeration of the
  output distribution at vocab 8 and gamma 3 (including a deliberately
  miscalibrated draft), and Monte Carlo agreement of the oracle's
  implementation with that enumeration (chi-square, and the acceptance rate
  against the closed form sum_v min(p, q); SPOT, "Experiments", validates its
  verifier the same way).
* tau in [1, gamma+1], counting the target's token (DFlash review,
  "Preliminary"); greedy known answers with planted matches.
* Gumbel-max draws follow softmax(z/T) (chi-square); shared-Gumbel coupling
  agreement is at least (1 - d)/(1 + d), d the total-variation distance
  (SPOT, "Coupled-noise verification").
"""

import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import stats

from oracle import philox
from oracle.drafter import lm_head
from oracle.verify import (FLAG_NEAR_TIE_TARGET, FLAG_ZERO_RESIDUAL, latency_per_token,
                           verify_batch, verify_greedy, verify_rs)


def _softmax(z):
    e = np.exp(z - z.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def enumerate_rs(p, q):
    """Exact outcome distribution of one speculative-sampling cycle, written
    from the algorithm's description: draft y_k ~ q_k, accept with probability
    min(1, p_k(y)/q_k(y)), at the first rejection emit a draw from
    norm(max(0, p_k - q_k)); after gamma acceptances emit a draw from p_gamma.
    Returns {emitted tuple: probability}."""
    gamma, V = q.shape
    out = {}

    def rec(k, prefix, prob):
        if k == gamma:
            for v in range(V):
                key = prefix + (v,)
                out[key] = out.get(key, 0.0) + prob * p[gamma][v]
            return
        r = np.maximum(p[k] - q[k], 0.0)
        rs = r.sum()
        for y in range(V):
            if q[k][y] == 0:
                continue
            a = min(1.0, p[k][y] / q[k][y])
            rec(k + 1, prefix + (y,), prob * q[k][y] * a)
            if a < 1.0:
                for v in range(V):
                    if r[v] > 0:
                        key = prefix + (v,)
                        out[key] = out.get(key, 0.0) + \
                            prob * q[k][y] * (1 - a) * r[v] / rs
    rec(0, (), 1.0)
    return out


def _cases():
    rng = np.random.default_rng(5)
    V, gamma = 8, 3
    zt = rng.normal(0, 1.5, (gamma + 1, V))
    close = zt[:gamma] + rng.normal(0, 0.3, (gamma, V))
    far = rng.normal(0, 2.5, (gamma, V))
    # miscalibrated: draft mass concentrated on tokens the target dislikes
    bad = -zt[:gamma] * 2.0
    return [(zt, close), (zt, far), (zt, bad)]


@pytest.mark.parametrize("case", range(3))
def test_rs_lossless_exact_enumeration(case):
    zt, zd = _cases()[case]
    p, q = _softmax(zt), _softmax(zd)
    gamma, V = q.shape
    dist = enumerate_rs(p, q)
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    # for every k <= gamma+1 and v_1..v_k: continuing with the target after
    # the cycle's tokens, the first k tokens follow prod_j p_j(v_j)
    for k in range(1, gamma + 2):
        for v in itertools.product(range(V), repeat=k):
            tot = 0.0
            for e, pe in dist.items():
                m = min(len(e), k)
                if e[:m] != v[:m]:
                    continue
                tail = 1.0
                for j in range(len(e), k):
                    tail *= p[j][v[j]]
                tot += pe * tail
            want = np.prod([p[j][v[j]] for j in range(k)])
            assert abs(tot - want) < 1e-12


@pytest.mark.parametrize("case", [0, 2])
def test_rs_implementation_matches_enumeration(case):
    zt, zd = _cases()[case]
    p, q = _softmax(zt), _softmax(zd)
    gamma, V = q.shape
    dist = enumerate_rs(p, q)
    rng = np.random.default_rng(100 + case)
    n = 60000
    counts = {}
    acc0 = 0
    for _ in range(n):
        y = np.array([rng.choice(V, p=q[k]) for k in range(gamma)])
        u = rng.random(gamma)
        g = rng.gumbel(size=(gamma + 1, V))
        toks, tau, _f = verify_rs(zt, zd, y, 1.0, u, lambda k: g[k])
        assert 1 <= tau <= gamma + 1 and len(toks) == tau
        counts[tuple(toks)] = counts.get(tuple(toks), 0) + 1
        acc0 += tau > 1
    # acceptance rate of the first draft token vs sum_v min(p, q)
    a_theory = np.minimum(p[0], q[0]).sum()
    se = np.sqrt(a_theory * (1 - a_theory) / n)
    assert abs(acc0 / n - a_theory) < max(5 * se, 0.002)
    # chi-square on (tau, first token, last token) cells
    cell_p, cell_n = {}, {}
    for e, pe in dist.items():
        key = (len(e), e[0], e[-1])
        cell_p[key] = cell_p.get(key, 0.0) + pe
    for e, c in counts.items():
        key = (len(e), e[0], e[-1])
        assert key in cell_p, f"impossible outcome {e}"
        cell_n[key] = cell_n.get(key, 0) + c
    keys = sorted(cell_p)
    exp_ = np.array([cell_p[k] * n for k in keys])
    obs = np.array([cell_n.get(k, 0) for k in keys], dtype=float)
    big = exp_ >= 5
    e2 = np.append(exp_[big], exp_[~big].sum())
    o2 = np.append(obs[big], obs[~big].sum())
    chi = stats.chisquare(o2, e2 * o2.sum() / e2.sum())
    assert chi.pvalue > 1e-4


def test_rs_identical_distributions_accept_all():
    rng = np.random.default_rng(1)
    zt = rng.normal(0, 2, (5, 50))
    zd = zt[:4].copy()
    y = rng.integers(0, 50, 4)
    u = np.full(4, 1 - 2.0 ** -24)          # largest uniform the stream yields
    toks, tau, f = verify_rs(zt, zd, y, 1.0, u, lambda k: np.zeros(50))
    assert tau == 5 and toks[:4] == list(y)


def test_rs_zero_residual_flag():
    # p == q at a rejected position: residual is empty -> draw from p, flag
    zt = np.zeros((2, 4))
    zt[0] = [0.0, 1.0, 2.0, 3.0]
    zd = zt[:1].copy()
    toks, tau, f = verify_rs(zt, zd, np.array([3]), 1.0, np.array([2.0]),
                             lambda k: np.array([0.0, 0.0, 0.0, 5.0]))
    assert tau == 1 and f & FLAG_ZERO_RESIDUAL and toks == [3]


def test_rs_one_hot_draft_accept_probability():
    # q = delta_y (draft certain): accept probability equals p(y)
    V = 6
    zt = np.log(np.array([[0.1, 0.2, 0.3, 0.1, 0.2, 0.1]] * 2))
    zd = np.full((1, V), -1e4)
    zd[0, 2] = 0.0
    n, acc = 20000, 0
    rng = np.random.default_rng(3)
    for _ in range(n):
        _t, tau, _f = verify_rs(zt, zd, np.array([2]), 1.0, rng.random(1),
                                lambda k: rng.gumbel(size=V))
        acc += tau == 2
    assert abs(acc / n - 0.3) < 5 * np.sqrt(0.3 * 0.7 / n)


def test_greedy_planted_matches():
    rng = np.random.default_rng(0)
    gamma, V = 15, 97
    zt = rng.normal(0, 2, (gamma + 1, V))
    t = np.argmax(zt, -1)
    for k in range(gamma + 1):
        y = rng.integers(0, V, gamma)
        y[:k] = t[:k]
        if k < gamma and y[k] == t[k]:
            y[k] = (t[k] + 1) % V
        toks, tau, f = verify_greedy(zt, y)
        assert tau == k + 1
        assert toks == list(t[:k]) + [int(t[k])]
        assert f == 0


def test_greedy_near_tie_flag():
    # a target row whose top-2 gap is below 1e-5 is flagged only when it
    # decides the outcome (rows 0..L)
    zt = np.zeros((3, 5))
    zt[0] = [0.0, 1.0, 0.2, 0.0, 0.0]
    zt[1] = [0.0, 0.5, 0.5 + 5e-6, 0.0, 0.0]
    zt[2] = [2.0, 0.0, 0.0, 0.0, 0.0]
    _t, tau, f = verify_greedy(zt, np.array([3, 2]))      # rejects at row 0
    assert tau == 1 and f == 0
    _t, tau, f = verify_greedy(zt, np.array([1, 2]))      # row 1 decides
    assert tau == 3 and f & FLAG_NEAR_TIE_TARGET


def test_greedy_lowest_index_tie():
    zt = np.array([[1.0, 3.0, 3.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    toks, tau, _ = verify_greedy(zt, np.array([2]))
    assert tau == 1 and toks == [1]
    toks, tau, _ = verify_greedy(zt, np.array([1]))
    assert tau == 2 and toks == [1, 0]


@settings(max_examples=40, deadline=None)
@given(gamma=st.integers(1, 15), V=st.integers(2, 40), seed=st.integers(0, 10**6),
       rs=st.booleans())
def test_tau_range_property(gamma, V, seed, rs):
    rng = np.random.default_rng(seed)
    bs = 3
    zt = rng.normal(0, 2, (bs, gamma + 1, V))
    zd = rng.normal(0, 2, (bs, gamma, V))
    y = rng.integers(0, V, (bs, gamma))
    toks, tau, flags = verify_batch("rs" if rs else "greedy", zt, y, zd=zd,
                                    seed=seed, cycle=seed % 7)
    for b in range(bs):
        assert 1 <= tau[b] <= gamma + 1
        assert np.all(toks[b, :tau[b]] >= 0) and np.all(toks[b, tau[b]:] == -1)
        assert list(toks[b, :tau[b] - 1]) == list(y[b, :tau[b] - 1])


def test_latency_identity():
    # DFlash review, "Preliminary": L = (T_draft + T_verify) / tau; speedup
    # eta = L_target / L.  tau counts the bonus token, so tau = 1 gives one
    # token per cycle and L is the whole cycle time.
    assert latency_per_token(4.0, 26.0, 1) == 30.0
    assert latency_per_token(4.0, 26.0, 6.0) == 5.0


def test_gumbel_max_follows_softmax():
    V, T = 12, 0.7
    rng = np.random.default_rng(9)
    z = rng.normal(0, 1.5, V)
    n = 30000
    g = philox.gumbel(4, philox.PURPOSE_DRAFT, 0, 0,
                      np.arange(n, dtype=np.uint64)[:, None],
                      np.arange(V, dtype=np.uint64)[None, :])
    out = lm_head(np.eye(V), np.tile(z, (n, 1)), temperature=T, gumbel=g)
    obs = np.bincount(out["ids"], minlength=V)
    p = _softmax(z / T)
    assert stats.chisquare(obs, p * n).pvalue > 1e-4


def test_shared_gumbel_coupling_bound():
    V = 10
    rng = np.random.default_rng(11)
    n = 20000
    g = philox.gumbel(1, philox.PURPOSE_SHARED, 0, 3,
                      np.arange(n, dtype=np.uint64)[:, None],
                      np.arange(V, dtype=np.uint64)[None, :])
    for scale in (0.2, 1.0, 3.0):
        a = rng.normal(0, 1, V)
        b = a + rng.normal(0, scale, V)
        P, Q = _softmax(a), _softmax(b)
        d = 0.5 * np.abs(P - Q).sum()
        x = lm_head(np.eye(V), np.tile(a, (n, 1)), gumbel=g)["ids"]
        y = lm_head(np.eye(V), np.tile(b, (n, 1)), gumbel=g)["ids"]
        agree = np.mean(x == y)
        assert agree >= (1 - d) / (1 + d) - 4 * np.sqrt(0.25 / n)
        # marginals are still exact draws from P and Q
        assert stats.chisquare(np.bincount(x, minlength=V), P * n).pvalue > 1e-4


# -- data faults: BAD_INPUT covers exactly the values the decisions read ------

def _rs_case(seed=3, gamma=4, V=12):
    rng = np.random.default_rng(seed)
    zt = rng.normal(0, 2, (gamma + 1, V))
    zd = rng.normal(0, 2, (gamma, V))
    y = rng.integers(0, V, gamma)
    u = np.full(gamma, 1e-3)          # every finite test accepts unless p/q tiny
    g = lambda k: philox.gumbel_row(0, philox.PURPOSE_RESIDUAL, 0, k, 0, V)
    return zt, zd, y, u, g


@pytest.mark.parametrize("where", ["target_bonus_row", "draft_at_y", "draft_lse", "rejected_row"])
def test_rs_bad_input_on_values_read(where):
    from oracle.verify import FLAG_BAD_INPUT
    zt, zd, y, u, g = _rs_case()
    if where == "target_bonus_row":
        zt[-1, 5] = np.nan                  # read by the last row's log-sum-exp
    elif where == "draft_at_y":
        zd[1, y[1]] = np.inf                # the accept test of slot 1 reads it
    elif where == "draft_lse":
        zd[2, (y[2] + 1) % 12] = np.nan     # not at y, but in the row's log-sum-exp
    else:
        zt[0, y[0]] = -30.0                 # slot 0 is rejected ...
        zd[0, (y[0] + 1) % 12] = -np.inf    # ... and the residual reads its whole row
    _, tau, f = verify_rs(zt, zd, y, 1.0, u, g)
    assert f & FLAG_BAD_INPUT and 1 <= tau <= 5


def test_rs_unread_infinite_draft_value_is_not_a_fault():
    """-inf in an accepted draft row away from y changes no value the
    decisions read (its row's log-sum-exp stays finite): no flag, and the
    same outcome as a very negative finite logit."""
    from oracle.verify import FLAG_BAD_INPUT
    zt, zd, y, u, g = _rs_case()
    zd2 = zd.copy()
    zd2[0, (y[0] + 1) % 12] = -np.inf
    zd3 = zd.copy()
    zd3[0, (y[0] + 1) % 12] = -1e300
    a = verify_rs(zt, zd2, y, 1.0, u, g)
    b = verify_rs(zt, zd3, y, 1.0, u, g)
    assert a[2] & FLAG_BAD_INPUT == 0 and a == b and a[1] >= 2


def test_rs_out_of_range_id_flagged_and_clamped():
    from oracle.verify import FLAG_BAD_INPUT
    zt, zd, y, u, g = _rs_case()
    y = y.copy()
    y[2] = 12                                # == V
    toks, tau, f = verify_rs(zt, zd, y, 1.0, u, g)
    assert f & FLAG_BAD_INPUT and all(0 <= t < 12 for t in toks) and 1 <= tau <= 5
