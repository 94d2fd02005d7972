"""GPU parity of dstill_verify against the oracle (oracle/verify.py).

The two sides get the same seeded inputs (synth.gen, drawn on the GPU and
copied to the host for the oracle).  Token ids and tau must agree bit-exactly
for every sequence that no near-tie flag marks on either side; flags
ZERO_RESIDUAL and BAD_INPUT must agree exactly.  Shapes: the tiny workload
(V 1024, gamma 7), a ragged vocabulary (V 5003, not a multiple of any split
or vector width), the full 8B-shaped vocabulary 151936 at gamma 15 with
batch 32 (bf16 target logits, N(0, 3), the bs-32 workload's rejection-
sampling configuration, the launch configuration the benchmark times), and
the degenerate gamma 1 / V 2.
"""

import numpy as np
import pytest
import torch

import block_diffusion_speculative_kv_amd as bd
from oracle import verify as ov
from oracle.drafter import logsumexp
from synth import gen
from tests.helpers import NEAR_BITS, compare_ids, device, to_np

pytestmark = pytest.mark.gpu


def _gpu_verify(mode, zt, y, zd=None, lse=None, T=1.0, seed=0, cycle=0):
    bs, g1, V = zt.shape
    dev = zt.device
    toks = torch.full((bs, g1), -7, dtype=torch.int32, device=dev)
    tau = torch.zeros(bs, dtype=torch.int32, device=dev)
    flags = torch.zeros(bs, dtype=torch.int32, device=dev)
    ws = torch.empty(bd.verify_workspace_bytes(bs, g1 - 1, V), dtype=torch.uint8, device=dev)
    bd.verify(mode, y, zt, toks, tau, flags, ws, temperature=T, seed=seed, cycle=cycle,
              draft_lse=lse, draft_logits=zd)
    torch.cuda.synchronize()
    return toks.cpu().numpy(), tau.cpu().numpy(), flags.cpu().numpy()


def _check(gpu, ref, what):
    gt, gtau, gf = gpu
    rt, rtau, rf = ref
    excl = ((gf & NEAR_BITS) != 0) | ((rf & NEAR_BITS) != 0)
    n = compare_ids(gtau, rtau, excl, what + " tau")
    compare_ids(gt, rt, np.repeat(excl[:, None], gt.shape[1], 1), what + " tokens")
    hard = 8 | 16
    assert np.array_equal(gf & hard, rf & hard), f"{what}: flags {gf} vs {rf}"
    return n


def _planted_greedy(zt_np, rng, gamma):
    """Draft ids matching the target's argmax for a planted prefix length."""
    bs = zt_np.shape[0]
    t = np.argmax(zt_np, -1)
    y = rng.integers(0, zt_np.shape[2], (bs, gamma))
    for b in range(bs):
        k = b % (gamma + 1)
        y[b, :k] = t[b, :k]
        if k < gamma and y[b, k] == t[b, k]:
            y[b, k] = (t[b, k] + 1) % zt_np.shape[2]
    return y


@pytest.mark.parametrize("bs,gamma,V,tdt", [(8, 7, 1024, "f32"), (17, 15, 5003, "f32"),
                                             (16, 15, 151936, "bf16"), (3, 1, 2, "f32")])
def test_greedy_parity(bs, gamma, V, tdt):
    dev = device()
    cfg = dict(bs=bs, gamma=gamma, vocab=V, target_logit_std=2.0, target_dtype=tdt, seed=11)
    zt = gen.target_logits(cfg, device=dev)
    zt_np = to_np(zt)
    rng = np.random.default_rng(bs * 1000 + gamma)
    y_np = _planted_greedy(zt_np, rng, gamma)
    y = torch.from_numpy(y_np.astype(np.int32)).to(dev)
    gpu = _gpu_verify(bd.VERIFY_GREEDY, zt, y)
    ref = ov.verify_batch("greedy", zt_np, y_np)
    # greedy verification does no arithmetic on the logits (argmax with the
    # lowest-id tie-break), so everything agrees exactly, flags included --
    # bf16 logits often hold exact top-2 ties, which both sides flag
    for g_, r_, name in zip(gpu, ref, ("tokens", "tau", "flags")):
        assert np.array_equal(g_, r_), f"greedy bs{bs} g{gamma} V{V}: {name} differ"
    # planted prefixes give every tau in 1..gamma+1
    assert sorted(set(gpu[1].tolist())) == sorted(set(ref[1].tolist()))


def test_greedy_bad_id_flagged():
    dev = device()
    cfg = dict(bs=2, gamma=4, vocab=300, target_logit_std=2.0, target_dtype="f32", seed=3)
    zt = gen.target_logits(cfg, device=dev)
    zt_np = to_np(zt)
    t = np.argmax(zt_np, -1)
    y_np = np.stack([t[0, :4], t[1, :4]]).astype(np.int64)
    y_np[1, 2] = 300          # out of the vocabulary: never matches, flagged
    y = torch.from_numpy(y_np.astype(np.int32)).to(dev)
    gpu = _gpu_verify(bd.VERIFY_GREEDY, zt, y)
    ref = ov.verify_batch("greedy", zt_np, y_np)
    _check(gpu, ref, "greedy bad id")
    assert gpu[1].tolist() == [5, 3]
    assert gpu[2][1] & bd.FLAG_BAD_INPUT and not gpu[2][0] & bd.FLAG_BAD_INPUT


def _rs_inputs(bs, gamma, V, tdt, kind, seed, std=3.0):
    dev = device()
    cfg = dict(bs=bs, gamma=gamma, vocab=V, target_logit_std=std, target_dtype=tdt, seed=seed)
    zt = gen.target_logits(cfg, device=dev)
    zt_np = to_np(zt)
    if kind == "independent":
        zd = gen.draft_logits(cfg, device=dev, std=std)
    elif kind == "equal":
        zd = zt[:, :gamma].float().contiguous()
    else:   # correlated: target plus N(0, 0.5) noise
        noise = gen.normal((bs, gamma, V), 0.5, seed=seed, name="draft_noise", device=dev)
        zd = (zt[:, :gamma].float() + noise).contiguous()
    zd_np = to_np(zd)
    return zt, zt_np, zd, zd_np


@pytest.mark.parametrize("bs,gamma,V,tdt,kind,T", [
    (32, 15, 151936, "bf16", "independent", 1.0),
    (32, 15, 151936, "bf16", "correlated", 1.0),
    (8, 15, 151936, "bf16", "equal", 1.0),
    (24, 7, 5003, "f32", "correlated", 0.7),
    (64, 3, 8, "f32", "correlated", 1.0),
    (4, 1, 2, "f32", "independent", 1.0),
])
def test_rs_parity(bs, gamma, V, tdt, kind, T):
    zt, zt_np, zd, zd_np = _rs_inputs(bs, gamma, V, tdt, kind, seed=bs + V)
    dev = zt.device
    # draft ids: a Gumbel-max draw from q (host numpy noise, any draw works)
    rng = np.random.default_rng(7)
    y_np = np.argmax(zd_np / T + rng.gumbel(size=zd_np.shape), -1)
    # draft log-normaliser at temperature T, from the oracle (fp64)
    lse_np = logsumexp(zd_np / T, axis=-1)
    y = torch.from_numpy(y_np.astype(np.int32)).to(dev)
    lse = torch.from_numpy(lse_np.astype(np.float32)).to(dev)
    seed, cycle = 1234, 5
    gpu = _gpu_verify(bd.VERIFY_RS, zt, y, zd=zd, lse=lse, T=T, seed=seed, cycle=cycle)
    ref = ov.verify_batch("rs", zt_np, y_np, zd=zd_np, temperature=T, seed=seed, cycle=cycle)
    n = _check(gpu, ref, f"rs {kind} bs{bs} g{gamma} V{V}")
    assert n <= max(1, bs // 8), f"{n} sequences flagged"
    assert np.all((gpu[1] >= 1) & (gpu[1] <= gamma + 1))
    if kind == "equal":
        # p == q: every draft token is accepted, the bonus comes from p_gamma
        assert np.all(gpu[1] == gamma + 1)


def test_rs_replays_with_same_counter_and_changes_with_cycle():
    zt, zt_np, zd, zd_np = _rs_inputs(8, 15, 5003, "f32", "correlated", seed=2)
    dev = zt.device
    y = torch.from_numpy(np.argmax(zd_np, -1).astype(np.int32)).to(dev)
    lse = torch.from_numpy(logsumexp(zd_np, axis=-1).astype(np.float32)).to(dev)
    a = _gpu_verify(bd.VERIFY_RS, zt, y, zd=zd, lse=lse, seed=9, cycle=1)
    b = _gpu_verify(bd.VERIFY_RS, zt, y, zd=zd, lse=lse, seed=9, cycle=1)
    c = _gpu_verify(bd.VERIFY_RS, zt, y, zd=zd, lse=lse, seed=9, cycle=2)
    for x, z in zip(a, b):
        assert np.array_equal(x, z)
    assert not all(np.array_equal(x, z) for x, z in zip(a, c))


@pytest.mark.parametrize("mode", ["greedy", "rs"])
def test_non_finite_inputs_flag_like_the_oracle(mode):
    """BAD_INPUT marks a non-finite value among the inputs the decisions read:
    any target logit; in rejection sampling also the draft logit of each
    slot's id, each draft row's log-sum-exp, and the whole draft row of the
    first rejection.  The flag must agree bit for bit; a flagged sequence's
    tokens are unspecified but tau stays in range; unflagged sequences agree
    as usual."""
    dev = device()
    bs, gamma, V = 10, 7, 5003
    tdt = "f32" if mode == "greedy" else "bf16"
    zt, zt_np, zd, zd_np = _rs_inputs(bs, gamma, V, tdt, "correlated", seed=41)
    zt_np = zt_np.copy()
    zd_np = zd_np.copy()
    rng = np.random.default_rng(3)
    y_np = np.argmax(zd_np + rng.gumbel(size=zd_np.shape), -1)
    if mode == "greedy":
        y_np[:, :3] = np.argmax(zt_np[:, :3], -1)   # a few accepted slots
    nan, inf = np.nan, np.inf
    zt_np[0, gamma, 17] = nan                        # target bonus row
    zt_np[1, 0, 4000] = inf                          # target row 0
    zt_np[2, 3, 5] = -inf                            # target row 3
    if mode == "rs":
        zd_np[3, 1, y_np[3, 1]] = inf                 # draft logit at y
        zd_np[4, 2, (y_np[4, 2] + 1) % V] = nan       # draft row 2's log-sum-exp
        zt_np[5, 0, y_np[5, 0]] = -60.0               # slot 0 rejected ...
        zd_np[5, 0, (y_np[5, 0] + 9) % V] = -inf      # ... its row holds -inf
        zd_np[7, 0, (y_np[7, 0] + 1) % V] = -inf      # away from y in an accepted row:
        zt_np[7, 0, y_np[7, 0]] = zd_np[7, 0, y_np[7, 0]] + 8.0   # unread, no flag
    zt_t = torch.from_numpy(zt_np).to(zt.dtype).to(dev)
    zt_np = to_np(zt_t)                              # what the kernel sees (bf16 rounding)
    y = torch.from_numpy(y_np.astype(np.int32)).to(dev)
    if mode == "greedy":
        gpu = _gpu_verify(bd.VERIFY_GREEDY, zt_t, y)
        ref = ov.verify_batch("greedy", zt_np, y_np)
    else:
        with np.errstate(invalid="ignore", over="ignore"):
            lse_np = logsumexp(zd_np, axis=-1)
        zd_t = torch.from_numpy(zd_np.astype(np.float32)).to(dev)
        lse = torch.from_numpy(lse_np.astype(np.float32)).to(dev)
        gpu = _gpu_verify(bd.VERIFY_RS, zt_t, y, zd=zd_t, lse=lse, seed=5, cycle=2)
        ref = ov.verify_batch("rs", zt_np, y_np, zd=zd_np.astype(np.float32).astype(np.float64),
                              seed=5, cycle=2)
    gbad = (gpu[2] & bd.FLAG_BAD_INPUT) != 0
    rbad = (ref[2] & bd.FLAG_BAD_INPUT) != 0
    assert np.array_equal(gbad, rbad), f"{mode}: BAD_INPUT {gbad.astype(int)} vs {rbad.astype(int)}"
    want_bad = [0, 1, 2] + ([3, 4, 5] if mode == "rs" else [])
    assert sorted(np.nonzero(gbad)[0].tolist()) == want_bad
    assert np.all((gpu[1] >= 1) & (gpu[1] <= gamma + 1))
    ok = ~gbad
    _check(tuple(x[ok] for x in gpu), tuple(x[ok] for x in ref), f"{mode} unflagged rows")
