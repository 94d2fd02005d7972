"""Plain definitions of greedy and rejection-sampling verification.  Test
infrastructure only.

* DStill, "Inference": greedy verification accepts draft tokens while they
  match the target's top-1; the standard rejection-sampling verifier keeps the
  target's sampling distribution; after a rejection the target supplies a
  correction token, and if every draft token is accepted it supplies a bonus
  token, which becomes the next anchor.
* DFlash review, "Preliminary": tau in [1, gamma+1] is the number of tokens a
  cycle yields, the target's token included.
* The acceptance test and the residual distribution are the textbook ones of
  speculative sampling (Leviathan et al.; Chen et al., both cited on the DStill
  and DFlash pages): accept draft y_k ~ q_k with probability
  min(1, p_k(y) / q_k(y)); at the first rejection draw from
  norm(max(0, p_k - q_k)); if all gamma are accepted draw the bonus from
  p_gamma.  Draws: the accept test uses uniform u_k; the residual and bonus
  use Gumbel-max (argmax of log-weight + Gumbel noise).

Indexing: target row k (k = 0..gamma) is the target's distribution for the
token after block slot k; draft row k (k = 0..gamma-1) is the drafter's
distribution for block slot k + 1, whose token is y[k].
"""

from __future__ import annotations

import numpy as np

from . import philox
from .drafter import logsumexp

NEAR = 1e-5

FLAG_NEAR_TIE_TARGET = 1      # target argmax top-2 gap below NEAR
FLAG_NEAR_THRESHOLD = 2       # |p/q - u| below NEAR at a deciding test
FLAG_NEAR_TIE_SAMPLE = 4      # residual / bonus Gumbel-max top-2 gap below NEAR
FLAG_ZERO_RESIDUAL = 8        # max(0, p - q) summed to zero: drew from p
FLAG_BAD_INPUT = 16           # draft id out of range or a non-finite logit read
# (tokens, tau and the other flags of a sequence flagged BAD_INPUT follow from
# the clamped ids and the non-finite values as they fall: unspecified)


def _argmax_gap(score):
    i = int(np.argmax(score))
    top = score[i]
    rest = np.delete(score, i)
    gap = top - (np.max(rest) if rest.size else -np.inf)
    return i, gap


def verify_greedy(zt, y):
    """zt [gamma+1, V] target logits, y [gamma] draft ids.
    Returns (tokens, tau, flags)."""
    zt = np.asarray(zt, dtype=np.float64)
    y = np.asarray(y)
    gamma = y.shape[0]
    flags = 0
    if np.any((y < 0) | (y >= zt.shape[1])) or not np.all(np.isfinite(zt)):
        flags |= FLAG_BAD_INPUT
    t = np.argmax(zt, axis=-1)
    L = 0
    while L < gamma and int(y[L]) == int(t[L]):
        L += 1
    # the target rows whose argmax decided the outcome are 0..L
    for k in range(L + 1):
        if _argmax_gap(zt[k])[1] < NEAR:
            flags |= FLAG_NEAR_TIE_TARGET
    tokens = [int(v) for v in y[:L]] + [int(t[L])]
    return tokens, L + 1, flags


def verify_rs(zt, zd, y, temperature, u, gumbel_at):
    """Rejection-sampling verification of one sequence.

    zt [gamma+1, V] target logits, zd [gamma, V] draft logits, y [gamma] draft
    ids, u [gamma] accept uniforms, gumbel_at(k) -> Gumbel noise [V] for the
    residual (k < gamma) or bonus (k = gamma) draw.  Returns
    (tokens, tau, flags)."""
    zt = np.asarray(zt, dtype=np.float64) / float(temperature)
    zd = np.asarray(zd, dtype=np.float64) / float(temperature)
    y = np.asarray(y)
    gamma = y.shape[0]
    flags = 0
    # Data faults: a draft id out of range, or a non-finite value among the
    # inputs the accept tests read -- any target logit (each row's
    # log-sum-exp needs all of it), and for every slot k the draft logit of
    # y_k and the draft row's log-sum-exp -- or in the draft row of the first
    # rejection (the residual reads all of it).
    bad = np.any((y < 0) | (y >= zt.shape[1])) or not np.all(np.isfinite(zt))
    lt = logsumexp(zt, axis=-1)
    with np.errstate(invalid="ignore", over="ignore"):
        ld = logsumexp(zd, axis=-1)
    yc = np.clip(y, 0, zt.shape[1] - 1)
    if not (np.all(np.isfinite(zd[np.arange(gamma), yc])) and np.all(np.isfinite(ld))):
        bad = True
    if bad:
        flags |= FLAG_BAD_INPUT
    for k in range(gamma):
        yk = int(yc[k])
        ratio = np.exp((zt[k, yk] - lt[k]) - (zd[k, yk] - ld[k]))
        if abs(ratio - u[k]) < NEAR:
            flags |= FLAG_NEAR_THRESHOLD
        if u[k] < ratio:
            continue
        if not np.all(np.isfinite(zd[k])):
            flags |= FLAG_BAD_INPUT
        p = np.exp(zt[k] - lt[k])
        q = np.exp(zd[k] - ld[k])
        r = np.maximum(p - q, 0.0)
        g = gumbel_at(k)
        if not np.any(r > 0):
            flags |= FLAG_ZERO_RESIDUAL
            score = np.log(p) + g
        else:
            with np.errstate(divide="ignore"):
                score = np.where(r > 0, np.log(r), -np.inf) + g
        v, gap = _argmax_gap(score)
        if gap < NEAR:
            flags |= FLAG_NEAR_TIE_SAMPLE
        return [int(t) for t in yc[:k]] + [v], k + 1, flags
    score = zt[gamma] - lt[gamma] + gumbel_at(gamma)
    v, gap = _argmax_gap(score)
    if gap < NEAR:
        flags |= FLAG_NEAR_TIE_SAMPLE
    return [int(t) for t in yc] + [v], gamma + 1, flags


def accept_uniforms(seed, seq, cycle, gamma):
    """u_k for k = 0..gamma-1 of one sequence (purpose 1, element 0)."""
    return philox.uniform(seed, philox.PURPOSE_ACCEPT, seq,
                          np.arange(gamma, dtype=np.uint64), cycle, 0)


def verify_batch(mode, zt, y, *, zd=None, temperature=1.0, seed=0, cycle=0):
    """Verify every sequence of a batch.  zt [bs, gamma+1, V], y [bs, gamma],
    zd [bs, gamma, V] (RS only).  Returns tokens [bs, gamma+1] (emitted ids,
    -1 after tau), tau [bs], flags [bs]."""
    zt = np.asarray(zt)
    bs, g1, V = zt.shape
    gamma = g1 - 1
    toks = np.full((bs, g1), -1, dtype=np.int64)
    taus = np.zeros(bs, dtype=np.int64)
    flags = np.zeros(bs, dtype=np.int64)
    for b in range(bs):
        if mode == "greedy":
            t, tau, f = verify_greedy(zt[b], y[b])
        else:
            u = accept_uniforms(seed, b, cycle, gamma)

            def g_at(k, b=b):
                return philox.gumbel_row(seed, philox.PURPOSE_RESIDUAL, b, k,
                                         cycle, V)
            t, tau, f = verify_rs(zt[b], zd[b], y[b], temperature, u, g_at)
        toks[b, :tau] = t
        taus[b] = tau
        flags[b] = f
    return toks, taus, flags


def latency_per_token(t_draft, t_verify, tau):
    """DFlash review, "Preliminary": L = (T_draft + T_verify) / tau."""
    return (t_draft + t_verify) / tau
