"""GPU parity of dstill_refine_commit (one pass of DStill's multi-step
refinement) against oracle.refine.

Cases:
* the whole K-pass schedule on seeded per-pass head statistics, K = 1, 4, 8
  and 15, block 16, with planted exact confidence ties and greedy ids equal
  to the mask id (the committed set is tracked by commit pass, not by
  token); tokens and commit passes bit-exact after every pass;
* a K = 4 rollout on the reduced bf16 drafter: each pass drafts the current
  block state and runs the greedy head on the GPU, then commits; the oracle
  applies its own commit step to the GPU's head outputs (shared inputs) and
  must agree bit-exactly, and the drafted logits of each pass are held to
  the drafter's 2e-2 bar against the oracle drafter on the same state.
"""

import numpy as np
import pytest
import torch

import block_diffusion_speculative_kv_amd as bd
import oracle.refine as orf
from oracle.drafter import Drafter as OracleDrafter
from synth import configs, gen
from tests.helpers import device, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [1, 4, 8, 15])
def test_schedule_on_synthetic_statistics(K):
    dev = device()
    rng = np.random.default_rng(K)
    bs, B, mask = 6, 16, 4999
    tokens = np.full((bs, B), mask, dtype=np.int64)
    tokens[:, 0] = rng.integers(0, 4999, bs)
    kappa = np.full((bs, B), -1, dtype=np.int64)
    kappa[:, 0] = 0
    tg = torch.tensor(tokens, dtype=torch.int32, device=dev)
    kg = torch.tensor(kappa, dtype=torch.int32, device=dev)
    for t in range(1, K + 1):
        ids = rng.integers(0, 5000, (bs, B - 1))
        ids[1, :] = mask  # greedy ids equal to the mask id
        zmax = rng.normal(0, 3, (bs, B - 1)).astype(np.float32)
        lse = (zmax + np.abs(rng.normal(0, 1, (bs, B - 1)))).astype(np.float32)
        zmax[2, 3], lse[2, 3] = zmax[2, 7], lse[2, 7]  # exact ties
        zmax[2, 9], lse[2, 9] = zmax[2, 7], lse[2, 7]
        tt = lambda a, dt: torch.tensor(a, dtype=dt, device=dev)
        bd.refine_commit(tt(ids, torch.int32), tt(zmax, torch.float32), tt(lse, torch.float32),
                         t, K, tg, kg)
        for b in range(bs):
            tokens[b], kappa[b] = orf.refine_step(tokens[b], kappa[b], ids[b],
                                                  zmax[b].astype(np.float64),
                                                  lse[b].astype(np.float64), t, K)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(tg), tokens), f"pass {t}: tokens"
        assert np.array_equal(to_np(kg), kappa), f"pass {t}: commit passes"
    assert (kappa >= 0).all()


def test_rollout_on_the_drafter():
    dev = device()
    K = 4
    cfg = configs.small_bf16(bs=2, ctx=[37, 300])
    B, d, g, mask = cfg["block"], cfg["hidden"], cfg["gamma"], cfg["mask_token_id"]
    w = gen.weights(cfg, device=dev)
    dr = bd.Drafter(cfg, w)
    cap = 320
    ks, vs = gen.kv_cache(cfg, cap, device=dev)
    kv = bd.KVCache(ks, [bd.KVCache.tile_v(v) for v in vs])
    ctx = torch.tensor(cfg["ctx_lens"], dtype=torch.int32, device=dev)
    bs = cfg["bs"]
    ws = dr.workspace(max_batch=bs, max_copies=1, max_ctx=cap - B, max_head_rows=bs * g)
    tok = gen.block_tokens(cfg, device=dev).view(bs, B).contiguous()
    kap = torch.full((bs, B), -1, dtype=torch.int32, device=dev)
    kap[:, 0] = 0
    hid = torch.empty((bs, 1, B, d), dtype=dr.tdtype, device=dev)
    rows = bs * g
    ids = torch.empty(rows, dtype=torch.int32, device=dev)
    zmax = torch.empty(rows, dtype=torch.float32, device=dev)
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    w_np = to_np(w)
    od = OracleDrafter(cfg, w_np)
    kn, vn = [to_np(k) for k in ks], [to_np(v) for v in vs]
    t_ref, k_ref = to_np(tok), to_np(kap)
    for t in range(1, K + 1):
        dr.block_draft(tok.view(bs, 1, B), ctx, cap - B, kv, hid, ws)
        dr.lm_head_argmax(hid.view(-1, d)[1:], rows, g, B, ids, ws, zmax=zmax, lse=lse)
        torch.cuda.synchronize()
        state = to_np(tok)
        assert np.array_equal(state, t_ref), f"pass {t}: state before the pass"
        i_, z_, l_ = (to_np(ids).reshape(bs, g), to_np(zmax).reshape(bs, g),
                      to_np(lse).reshape(bs, g))
        for b, S in enumerate(cfg["ctx_lens"]):
            want = od.draft([k[b] for k in kn], [v[b] for v in vn], state[b][None], S)
            zg = to_np(hid)[b, 0, 1:] @ w_np["lm_head"].T
            zr = want[0, 1:] @ w_np["lm_head"].T
            assert np.abs(zg - zr).max() <= 2e-2, f"pass {t} seq {b}: logits"
            t_ref[b], k_ref[b] = orf.refine_step(t_ref[b], k_ref[b], i_[b], z_[b], l_[b], t, K)
        bd.refine_commit(ids.view(bs, g), zmax.view(bs, g), lse.view(bs, g), t, K, tok, kap)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(tok), t_ref) and np.array_equal(to_np(kap), k_ref)
    assert (to_np(kap) >= 0).all()


@pytest.mark.parametrize("B,K", [(2, 1), (64, 5), (64, 63)])
def test_block_size_edges(B, K):
    # gamma = 1; the largest block the kernel takes, with few and with B - 1 passes
    dev = device()
    rng = np.random.default_rng(B + K)
    bs, mask = 3, 4999
    tokens = np.full((bs, B), mask, dtype=np.int64)
    tokens[:, 0] = 1
    kappa = np.full((bs, B), -1, dtype=np.int64)
    kappa[:, 0] = 0
    tg = torch.tensor(tokens, dtype=torch.int32, device=dev)
    kg = torch.tensor(kappa, dtype=torch.int32, device=dev)
    for t in range(1, K + 1):
        ids = rng.integers(0, 5000, (bs, B - 1))
        zmax = rng.normal(0, 3, (bs, B - 1)).astype(np.float32)
        lse = (zmax + np.abs(rng.normal(0, 1, (bs, B - 1)))).astype(np.float32)
        tt = lambda a, dt: torch.tensor(a, dtype=dt, device=dev)
        bd.refine_commit(tt(ids, torch.int32), tt(zmax, torch.float32), tt(lse, torch.float32),
                         t, K, tg, kg)
        for b in range(bs):
            tokens[b], kappa[b] = orf.refine_step(tokens[b], kappa[b], ids[b],
                                                  zmax[b].astype(np.float64),
                                                  lse[b].astype(np.float64), t, K)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(tg), tokens) and np.array_equal(to_np(kg), kappa)
    assert (kappa >= 0).all()
