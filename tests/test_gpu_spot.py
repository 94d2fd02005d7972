"""GPU parity of dstill_spot_verify against oracle.spot.verify_tree.

Cases:
* seeded draft trees over synthetic per-slot head outputs (fp32): drafts
  that are their parent's true next state and drafts that are not, chains
  and fans, duplicate drafted states, a full block (no masked slot), parents
  that are not earlier states, planted exact ties in the slot confidence
  (zmax and lse copied between two masked slots), at T = 1 and T = 0.7;
  commits, count, deepest state and flags bit-exact (both sides rank the
  same fp32 statistics by the same fp64 expression);
* the multi-copy layout on the reduced bf16 drafter: the root and 8 drafted
  states drafted as 9 copies behind the shared context, the shared-Gumbel
  head over every slot, then the verification; the oracle verifies the
  GPU's head outputs (shared inputs), bit-exact.
"""

import numpy as np
import pytest
import torch

import block_diffusion_speculative_kv_amd as bd
import oracle.spot as osp
from synth import configs, gen
from tests.helpers import device, to_np

pytestmark = pytest.mark.gpu

MASK = 5002


def _tree(rng, L, n, ids, zmax, lse, T, root):
    states, parent = [root.copy()], [-1]
    for j in range(1, n):
        p = int(rng.integers(0, j))
        ps = states[p]
        m = np.flatnonzero(ps == MASK)
        u = rng.random()
        if m.size and u < 0.6:
            s, v, _ = osp.commit(ps, ids[p], zmax[p], lse[p], MASK, T)
            st = osp.apply(ps, s, v)
        elif m.size and u < 0.85:
            st = osp.apply(ps, int(rng.choice(m)), int(rng.integers(0, 5000)))
        else:
            st = ps.copy()
        states.append(st)
        parent.append(p)
    return np.stack(states), np.array(parent)


def _run(states, parent, ids, zmax, lse, gap, T, dev):
    bs, n, L = states.shape
    t = lambda a, dt: torch.tensor(np.ascontiguousarray(a), dtype=dt, device=dev)
    o_n = torch.empty(bs, dtype=torch.int32, device=dev)
    o_s = torch.empty((bs, n), dtype=torch.int32, device=dev)
    o_t = torch.empty((bs, n), dtype=torch.int32, device=dev)
    o_st = torch.empty(bs, dtype=torch.int32, device=dev)
    o_f = torch.empty(bs, dtype=torch.int32, device=dev)
    bd.spot_verify(t(states, torch.int32), t(parent, torch.int32), t(ids, torch.int32),
                   t(zmax, torch.float32), t(lse, torch.float32), MASK, o_n, o_s, o_t, o_st, o_f,
                   temperature=T, gap=None if gap is None else t(gap, torch.float32))
    torch.cuda.synchronize()
    return to_np(o_n), to_np(o_s), to_np(o_t), to_np(o_st), to_np(o_f)


def _check(states, parent, ids, zmax, lse, gap, T, got):
    o_n, o_s, o_t, o_st, o_f = got
    for b in range(states.shape[0]):
        commits, deepest, flags = osp.verify_tree(
            states[b], parent[b], ids[b], zmax[b].astype(np.float32).astype(np.float64),
            lse[b].astype(np.float32).astype(np.float64), MASK, np.float32(T),
            None if gap is None else gap[b].astype(np.float32))
        n = len(commits)
        assert o_n[b] == n, f"seq {b}: {o_n[b]} commits, oracle {n}"
        assert [(int(s), int(t)) for s, t in zip(o_s[b][:n], o_t[b][:n])] == commits, f"seq {b}"
        assert np.all(o_s[b][n:] == -1) and np.all(o_t[b][n:] == -1)
        assert (o_st[b], o_f[b]) == (deepest, flags), f"seq {b}: state/flags"


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_synthetic_trees(T):
    dev = device()
    rng = np.random.default_rng(7)
    bs, n, L = 12, 9, 16
    ids = rng.integers(0, 5000, (bs, n, L))
    zmax = rng.normal(0, 3, (bs, n, L)).astype(np.float32)
    lse = (zmax + np.abs(rng.normal(0, 1, (bs, n, L)))).astype(np.float32)
    gap = np.abs(rng.normal(0, 1, (bs, n, L))).astype(np.float32)
    gap[3, :, :] = 1e-6  # every commit of sequence 3 is a near-tie sample
    states, parent = [], []
    for b in range(bs):
        root = np.full(L, MASK)
        root[0] = int(rng.integers(0, 5000))
        if b == 1:
            root[:] = rng.integers(0, 5000, L)  # a full block: nothing to commit
        if b == 2:  # planted tie at the root's best slot
            k = 1 + int(np.argmax(zmax[b, 0, 1:] - lse[b, 0, 1:]))
            j = 1 + (k % (L - 1))
            zmax[b, 0, j], lse[b, 0, j] = zmax[b, 0, k], lse[b, 0, k]
        s_, p_ = _tree(rng, L, n, ids[b], zmax[b], lse[b], T, root)
        if b == 4:
            p_[5] = 7   # a parent that is not an earlier state
            p_[6] = -1
        if b == 5:
            s_[2] = s_[1]
            p_[2] = p_[1]  # a duplicate drafted state
        states.append(s_)
        parent.append(p_)
    states, parent = np.stack(states), np.stack(parent)
    got = _run(states, parent, ids, zmax, lse, gap, T, dev)
    _check(states, parent, ids, zmax, lse, gap, T, got)
    assert got[0].max() >= 3, "some drafts must be accepted"


def test_multicopy_layout_end_to_end():
    dev = device()
    D = 8
    cfg = configs.small_bf16(bs=2, ctx=[37, 300], n_copies=1 + D, lm_mode="shared_gumbel")
    B, d, V = cfg["block"], cfg["hidden"], cfg["vocab"]
    mask = cfg["mask_token_id"]
    w = gen.weights(cfg, device=dev)
    dr = bd.Drafter(cfg, w)
    cap = 320
    ks, vs = gen.kv_cache(cfg, cap, device=dev)
    kv = bd.KVCache(ks, [bd.KVCache.tile_v(v) for v in vs])
    ctx = torch.tensor(cfg["ctx_lens"], dtype=torch.int32, device=dev)
    bs, C = cfg["bs"], 1 + D
    rng = np.random.default_rng(9)
    # root (anchor + masks) and a draft tree of single-slot extensions
    states, parent = [], []
    for b in range(bs):
        root = np.full(B, mask)
        root[0] = int(rng.integers(0, V - 1))
        st, pa = [root], [-1]
        for j in range(1, C):
            p = int(rng.integers(0, j))
            m = np.flatnonzero(st[p] == mask)
            st.append(osp.apply(st[p], int(rng.choice(m)), int(rng.integers(0, V - 1))))
            pa.append(p)
        states.append(np.stack(st))
        parent.append(pa)
    states, parent = np.stack(states), np.array(parent)
    tok = torch.tensor(states, dtype=torch.int32, device=dev)
    ws = dr.workspace(max_batch=bs, max_copies=C, max_ctx=cap - B, max_head_rows=bs * C * B)
    hid = torch.empty((bs, C, B, d), dtype=dr.tdtype, device=dev)
    dr.block_draft(tok, ctx, cap - B, kv, hid, ws)
    rows = bs * C * B
    ids = torch.empty(rows, dtype=torch.int32, device=dev)
    zmax = torch.empty(rows, dtype=torch.float32, device=dev)
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    gap = torch.empty(rows, dtype=torch.float32, device=dev)
    dr.lm_head_argmax(hid.view(-1, d), rows, B, B, ids, ws, mode=bd.HEAD_SHARED_GUMBEL,
                      temperature=1.0, seed=3, cycle=1, zmax=zmax, lse=lse, gap=gap)
    torch.cuda.synchronize()
    sh = (bs, C, B)
    i_, z_, l_, g_ = (to_np(ids).reshape(sh), to_np(zmax).reshape(sh), to_np(lse).reshape(sh),
                      to_np(gap).reshape(sh))
    got = _run(states, parent, i_, z_, l_, g_, 1.0, dev)
    _check(states, parent, i_, z_, l_, g_, 1.0, got)


@pytest.mark.parametrize("n,L", [(1, 16), (64, 64), (5, 1)])
def test_tree_size_edges(n, L):
    # root only; the largest tree and block the kernel takes; a one-slot block
    dev = device()
    rng = np.random.default_rng(n * 100 + L)
    bs = 3
    ids = rng.integers(0, 5000, (bs, n, L))
    zmax = rng.normal(0, 3, (bs, n, L)).astype(np.float32)
    lse = (zmax + np.abs(rng.normal(0, 1, (bs, n, L)))).astype(np.float32)
    states, parent = [], []
    for b in range(bs):
        root = np.full(L, MASK)
        s_, p_ = _tree(rng, L, n, ids[b], zmax[b], lse[b], 1.0, root)
        states.append(s_)
        parent.append(p_)
    states, parent = np.stack(states), np.stack(parent)
    got = _run(states, parent, ids, zmax, lse, None, 1.0, dev)
    _check(states, parent, ids, zmax, lse, None, 1.0, got)
