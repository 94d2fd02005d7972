"""The planted-acceptance draw of the measurement harness (host code, no
GPU): accepted-prefix lengths k follow the truncated geometric law
P(k) = alpha^k (1 - alpha) for k < gamma and alpha^gamma at k = gamma, so
E[tau] = E[k] + 1 = 1 + sum_{j=1..gamma} alpha^j (6.50 at alpha 0.86,
gamma 15); the draw is a function of (seed, cycle) and differs across
cycles."""

import numpy as np

from block_diffusion_speculative_kv_amd.cycle import Cycle


class _Stub:
    seed, gamma, cfg = 0, 15, {"bs": 32}


def test_law_and_mean():
    s = _Stub()
    ks = np.concatenate([Cycle.plant_draw(s, c, 0.86) for c in range(4000)])
    n = ks.size
    assert ks.min() >= 0 and ks.max() <= 15
    p = np.array([0.86 ** k * 0.14 for k in range(15)] + [0.86 ** 15])
    assert abs(p.sum() - 1) < 1e-12
    freq = np.bincount(ks, minlength=16) / n
    # 5 standard errors per cell
    assert np.all(np.abs(freq - p) <= 5 * np.sqrt(p * (1 - p) / n))
    tau = 1 + sum(0.86 ** j for j in range(1, 16))
    assert abs(tau - 6.5033) < 1e-4
    assert abs((ks + 1).mean() - tau) <= 5 * (ks + 1).std() / np.sqrt(n)


def test_replay_and_cycle_dependence():
    s = _Stub()
    assert np.array_equal(Cycle.plant_draw(s, 7, 0.86), Cycle.plant_draw(s, 7, 0.86))
    assert not np.array_equal(Cycle.plant_draw(s, 7, 0.86), Cycle.plant_draw(s, 8, 0.86))


def test_extremes():
    s = _Stub()
    assert np.all(Cycle.plant_draw(s, 1, 1.0) == 15)   # every position accepted
    assert np.all(Cycle.plant_draw(s, 1, 0.0) == 0)    # none accepted
