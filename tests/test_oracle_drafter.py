"""Pins for the oracle's drafter (fusion, injection, block draft, LM head).

What fixes each part, other than the oracle itself:
* bfloat16 rounding: torch's float32 -> bfloat16 conversion (library routine).
* RMSNorm: torch.nn.functional.rms_norm; closed forms (constant vector, scale
  invariance).
* Rotary embedding: the complex-number form (x1 + i x2) e^{i pos w}; norm
  preservation; relative-position property of the scores.
* Block attention: the DFlash training formulation -- several blocks in one
  pass over the whole sequence with an explicit block-sparse mask (each block
  sees the clean context before its anchor and itself) -- must equal the
  inference formulation with injected K/V (DFlash review, "Method / Training"
  vs "Method / Inference"); evaluated with torch's scaled_dot_product_attention.
* Whole layer: an independent composition of torch library routines.
* Multi-copy isolation: copy c equals a run of copy c alone (SPOT, "Method").
* Injection: row independence (incremental == all at once, permutation).
* Position wiring: without rotary embedding and with no context all masked rows
  are identical; a common shift of every position changes nothing.
* LM head: log-sum-exp vs scipy.special.logsumexp; lowest-id tie-break.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp as sp_lse

import oracle.drafter as od
from synth import configs, gen


def _tiny(**kw):
    base = dict(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                mlp=96, vocab=50, n_feat_layers=3, target_hidden=32, gamma=5,
                dtype="f32", rms_eps=1e-6, rope_theta=1e4, qk_norm=1, bs=1,
                ctx=[9], n_copies=1, verify="greedy", lm_mode="argmax",
                temperature=1.0, target_logit_std=2.0, target_dtype="f32",
                seed=3)
    base.update(kw)
    return configs.finish(base, "tiny_test")


def _np(w):
    if isinstance(w, dict):
        return {k: _np(v) for k, v in w.items()}
    if isinstance(w, list):
        return [_np(v) for v in w]
    return w.float().numpy().astype(np.float64)


def _model(cfg):
    w = _np(gen.weights(cfg))
    # make weights larger than N(0, 0.02) so attention is far from uniform
    for lw in w["layers"]:
        lw["wqkv"] *= 10
    return od.Drafter(cfg, w), w


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.normal(0, 3, 100000).astype(np.float32)
    # exact ties between two bfloat16 neighbours
    ties = (rng.integers(0x0080, 0x7F00, 1000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = od.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want.astype(np.float64))


def test_rms_norm_pins():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 2, (7, 33))
    g = rng.normal(1, 0.1, 33)
    ref = F.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), eps=1e-6)
    assert np.allclose(od.rms_norm(x, g, 1e-6), ref.numpy(), rtol=1e-13, atol=0)
    c = np.full((1, 8), -2.5)
    assert np.allclose(od.rms_norm(c, np.ones(8), 0.0), -1.0, rtol=1e-15)
    assert np.allclose(od.rms_norm(x * 7.0, g, 0.0), od.rms_norm(x, g, 0.0),
                       rtol=1e-13)


def test_rope_pins():
    rng = np.random.default_rng(2)
    dh, theta = 16, 1e4
    x = rng.normal(0, 1, (5, 3, dh))
    pos = np.array([0, 1, 7, 100, 32767])
    y = od.rope(x, pos, theta)
    # complex form
    w = theta ** (-np.arange(dh // 2) * 2.0 / dh)
    zc = (x[..., :dh // 2] + 1j * x[..., dh // 2:]) * np.exp(1j * pos[:, None, None] * w)
    assert np.allclose(y[..., :dh // 2], zc.real, atol=1e-12)
    assert np.allclose(y[..., dh // 2:], zc.imag, atol=1e-12)
    assert np.allclose(y[0], x[0])                      # position 0 is identity
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    # scores depend only on the position difference
    q, k = rng.normal(0, 1, (1, 1, dh)), rng.normal(0, 1, (1, 1, dh))
    s1 = (od.rope(q, [10], theta) * od.rope(k, [3], theta)).sum()
    s2 = (od.rope(q, [1007], theta) * od.rope(k, [1000], theta)).sum()
    assert abs(s1 - s2) < 1e-9


def _torch_rope(x, pos, theta):
    dh = x.shape[-1]
    w = theta ** (-torch.arange(dh // 2, dtype=torch.float64) * 2.0 / dh)
    rot = torch.polar(torch.ones(len(pos), dh // 2, dtype=torch.float64),
                      torch.tensor(pos, dtype=torch.float64)[:, None] * w)
    z = torch.complex(x[..., :dh // 2], x[..., dh // 2:]) * rot[:, None, :]
    return torch.cat([z.real, z.imag], -1)


def _torch_draft(cfg, w, ctx_k, ctx_v, tokens, S):
    """Independent composition of torch library routines (fp64)."""
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    C, B = tokens.shape
    hq, hkv, dh, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["hidden"]
    eps = cfg["rms_eps"]
    h = F.embedding(torch.from_numpy(tokens.reshape(-1)).long(), T(w["embed"]))
    pos = [S + s for _ in range(C) for s in range(B)]
    for li, lw in enumerate(w["layers"]):
        u = F.rms_norm(h, (d,), T(lw["attn_norm"]), eps)
        q, k, v = F.linear(u, T(lw["wqkv"])).split([hq * dh, hkv * dh, hkv * dh], -1)
        q = _torch_rope(F.rms_norm(q.view(-1, hq, dh), (dh,), T(lw["q_norm"]), eps), pos, cfg["rope_theta"])
        k = _torch_rope(F.rms_norm(k.view(-1, hkv, dh), (dh,), T(lw["k_norm"]), eps), pos, cfg["rope_theta"])
        v = v.reshape(-1, hkv, dh)
        outs = []
        for c in range(C):
            sl = slice(c * B, (c + 1) * B)
            K = torch.cat([T(ctx_k[li])[:, :S], k[sl].transpose(0, 1)], 1)
            Vv = torch.cat([T(ctx_v[li])[:, :S], v[sl].transpose(0, 1)], 1)
            o = F.scaled_dot_product_attention(q[sl].transpose(0, 1)[None], K[None],
                                               Vv[None], enable_gqa=True)
            outs.append(o[0].transpose(0, 1).reshape(B, hq * dh))
        h = h + F.linear(torch.cat(outs, 0), T(lw["wo"]))
        u = F.rms_norm(h, (d,), T(lw["mlp_norm"]), eps)
        g, up = F.linear(u, T(lw["w_gate_up"])).chunk(2, -1)
        h = h + F.linear(F.silu(g) * up, T(lw["w_down"]))
    return F.rms_norm(h, (d,), T(w["g_final"]), eps).view(C, B, d).numpy()


@pytest.mark.parametrize("S,C", [(9, 1), (0, 1), (13, 3)])
def test_draft_matches_torch_composition(S, C):
    cfg = _tiny(n_copies=C)
    m, w = _model(cfg)
    rng = np.random.default_rng(4)
    feats = rng.normal(0, 1, (max(S, 1), cfg["feat_dim"]))
    ks, vs = m.inject_rows(feats, np.arange(max(S, 1)))
    ctx_k = [k.transpose(1, 0, 2) for k in ks]
    ctx_v = [v.transpose(1, 0, 2) for v in vs]
    tokens = np.full((C, cfg["block"]), cfg["mask_token_id"])
    tokens[:, 0] = 7
    if C > 1:
        tokens[1:, 2] = rng.integers(0, 49, C - 1)
    got = m.draft(ctx_k, ctx_v, tokens, S)
    want = _torch_draft(cfg, w, ctx_k, ctx_v, tokens, S)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10)


def test_injection_matches_torch():
    cfg = _tiny()
    m, w = _model(cfg)
    rng = np.random.default_rng(5)
    feats = rng.normal(0, 1, (6, cfg["feat_dim"]))
    pos = np.array([0, 5, 2, 9, 100, 3])
    ks, vs = m.inject_rows(feats, pos)
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    ht = F.rms_norm(F.linear(T(feats), T(w["w_fuse"])), (cfg["hidden"],), T(w["g_fuse"]), 1e-6)
    qd, kvd, dh = cfg["q_dim"], cfg["kv_dim"], cfg["head_dim"]
    for li, lw in enumerate(w["layers"]):
        wk = T(lw["wqkv"])[qd:qd + kvd]
        wv = T(lw["wqkv"])[qd + kvd:]
        k = F.rms_norm(F.linear(ht, wk).view(6, -1, dh), (dh,), T(lw["k_norm"]), 1e-6)
        k = _torch_rope(k, list(pos), cfg["rope_theta"])
        assert np.allclose(ks[li], k.numpy(), atol=1e-12)
        assert np.allclose(vs[li], F.linear(ht, wv).view(6, -1, dh).numpy(), atol=1e-12)


def test_training_mask_formulation_equals_injection():
    """Two blocks drafted in one pass over [context; block A; block B] with the
    block-sparse training mask equal two separate inference passes."""
    cfg = _tiny(n_layers=1)
    m, w = _model(cfg)
    rng = np.random.default_rng(6)
    N = 20
    SA, SB = 8, 17
    feats = rng.normal(0, 1, (N, cfg["feat_dim"]))
    ks, vs = m.inject_rows(feats, np.arange(N))
    ck = [k.transpose(1, 0, 2) for k in ks]
    cv = [v.transpose(1, 0, 2) for v in vs]
    B = cfg["block"]
    tA = np.array([[4] + [cfg["mask_token_id"]] * (B - 1)])
    tB = np.array([[11] + [cfg["mask_token_id"]] * (B - 1)])
    trA, trB = [], []
    m.draft(ck, cv, tA, SA, trace=trA)
    m.draft(ck, cv, tB, SB, trace=trB)
    hq, hkv, dh = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    q = np.concatenate([trA[0]["q"][0], trB[0]["q"][0]], 0)       # [2B, hq, dh]
    kk = np.concatenate([ks[0], trA[0]["k"][0], trB[0]["k"][0]], 0)  # [N+2B, hkv, dh]
    vv = np.concatenate([vs[0], trA[0]["v"][0], trB[0]["v"][0]], 0)
    mask = np.zeros((2 * B, N + 2 * B), dtype=bool)
    mask[:B, :SA] = True
    mask[:B, N:N + B] = True
    mask[B:, :SB] = True
    mask[B:, N + B:] = True
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    o = F.scaled_dot_product_attention(T(q.transpose(1, 0, 2))[None],
                                       T(kk.transpose(1, 0, 2))[None],
                                       T(vv.transpose(1, 0, 2))[None],
                                       attn_mask=T(mask)[None, None], enable_gqa=True)
    o = o[0].transpose(0, 1).reshape(2 * B, hq * dh).numpy()
    assert np.allclose(o[:B], trA[0]["attn"], atol=1e-12)
    assert np.allclose(o[B:], trB[0]["attn"], atol=1e-12)


def test_copy_isolation():
    cfg = _tiny(n_copies=4)
    m, _ = _model(cfg)
    rng = np.random.default_rng(7)
    S = 11
    ks, vs = m.inject_rows(rng.normal(0, 1, (S, cfg["feat_dim"])), np.arange(S))
    ck = [k.transpose(1, 0, 2) for k in ks]
    cv = [v.transpose(1, 0, 2) for v in vs]
    toks = rng.integers(0, 49, (4, cfg["block"]))
    allc = m.draft(ck, cv, toks, S)
    for c in range(4):
        one = m.draft(ck, cv, toks[c:c + 1], S)
        assert np.allclose(allc[c], one[0], rtol=1e-13, atol=1e-13)


def test_injection_row_independence():
    cfg = _tiny()
    m, _ = _model(cfg)
    rng = np.random.default_rng(8)
    feats = rng.normal(0, 1, (10, cfg["feat_dim"]))
    pos = np.arange(10)
    k_all, v_all = m.inject_rows(feats, pos)
    k1, v1 = m.inject_rows(feats[:3], pos[:3])
    k2, v2 = m.inject_rows(feats[3:], pos[3:])
    perm = rng.permutation(10)
    kp, vp = m.inject_rows(feats[perm], pos[perm])
    for li in range(cfg["n_layers"]):
        assert np.allclose(k_all[li], np.concatenate([k1[li], k2[li]]), rtol=1e-13)
        assert np.allclose(v_all[li], np.concatenate([v1[li], v2[li]]), rtol=1e-13)
        assert np.allclose(k_all[li][perm], kp[li], rtol=1e-13)
        assert np.allclose(v_all[li][perm], vp[li], rtol=1e-13)


def test_position_wiring(monkeypatch):
    cfg = _tiny()
    m, _ = _model(cfg)
    B = cfg["block"]
    empty = [np.zeros((cfg["n_kv_heads"], 0, cfg["head_dim"]))] * cfg["n_layers"]
    toks = np.array([[5] + [cfg["mask_token_id"]] * (B - 1)])
    with_rope = m.draft(empty, empty, toks, 0)[0]
    assert not np.allclose(with_rope[1], with_rope[2])
    monkeypatch.setattr(od, "rope", lambda x, pos, theta: np.asarray(x, dtype=np.float64))
    no_rope = m.draft(empty, empty, toks, 0)[0]
    for s in range(2, B):
        assert np.allclose(no_rope[s], no_rope[1], rtol=1e-13, atol=1e-13)


def test_common_position_shift_is_invisible(monkeypatch):
    cfg = _tiny()
    m, _ = _model(cfg)
    rng = np.random.default_rng(9)
    S = 7
    feats = rng.normal(0, 1, (S, cfg["feat_dim"]))
    toks = np.array([[3] + [cfg["mask_token_id"]] * (cfg["block"] - 1)])

    def run():
        ks, vs = m.inject_rows(feats, np.arange(S))
        return m.draft([k.transpose(1, 0, 2) for k in ks],
                       [v.transpose(1, 0, 2) for v in vs], toks, S)
    base = run()
    real = od.rope
    monkeypatch.setattr(od, "rope", lambda x, pos, theta: real(x, np.asarray(pos) + 1000, theta))
    shifted = run()
    assert np.allclose(base, shifted, rtol=1e-8, atol=1e-9)


def test_lm_head_pins():
    rng = np.random.default_rng(10)
    hid = rng.normal(0, 1, (5, 16))
    W = rng.normal(0, 0.5, (40, 16))
    out = od.lm_head(W, hid, temperature=0.8, keep_logits=True)
    z = hid @ W.T
    assert np.allclose(out["lse"], sp_lse(z / 0.8, axis=-1), rtol=1e-13)
    assert np.array_equal(out["ids"], np.argmax(z, -1))
    assert np.allclose(out["zsel"], z.max(-1))
    # ties: lowest id wins, gap 0
    W2 = np.zeros((6, 2))
    W2[2] = W2[4] = [1, 0]
    o2 = od.lm_head(W2, np.array([[1.0, 0.0]]))
    assert o2["ids"][0] == 2 and o2["gap"][0] == 0.0


@pytest.mark.parametrize("S,W", [(20, 6), (20, 19), (5, 8)])
def test_sliding_window_matches_explicit_mask(S, W):
    """The windowed layer's attention equals SDPA over [context; block] with
    the mask that lets the block see context positions [S - W, S) and itself;
    a layer whose full-attention bit is set, and a window of at least S, give
    the unwindowed result."""
    cfg = _tiny(n_layers=2, swa_window=W, full_attn_mask=0b10)
    m, w = _model(cfg)
    rng = np.random.default_rng(11)
    feats = rng.normal(0, 1, (S, cfg["feat_dim"]))
    ks, vs = m.inject_rows(feats, np.arange(S))
    ck = [k.transpose(1, 0, 2) for k in ks]
    cv = [v.transpose(1, 0, 2) for v in vs]
    B = cfg["block"]
    tok = np.array([[4] + [cfg["mask_token_id"]] * (B - 1)])
    tr = []
    m.draft(ck, cv, tok, S, trace=tr)
    hq, dh = cfg["n_q_heads"], cfg["head_dim"]
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    for li in (0, 1):
        q = tr[li]["q"][0]
        kk = np.concatenate([ks[li], tr[li]["k"][0]], 0)
        vv = np.concatenate([vs[li], tr[li]["v"][0]], 0)
        mask = np.zeros((B, S + B), dtype=bool)
        lo = max(0, S - W) if li == 0 else 0
        mask[:, lo:S] = True
        mask[:, S:] = True
        o = F.scaled_dot_product_attention(T(q.transpose(1, 0, 2))[None],
                                           T(kk.transpose(1, 0, 2))[None],
                                           T(vv.transpose(1, 0, 2))[None],
                                           attn_mask=T(mask)[None, None], enable_gqa=True)
        o = o[0].transpose(0, 1).reshape(B, hq * dh).numpy()
        assert np.allclose(o, tr[li]["attn"], atol=1e-12)
    if W >= S:
        full = _tiny(n_layers=2)
        mf, _ = _model(full)
        assert np.allclose(mf.draft(ck, cv, tok, S), m.draft(ck, cv, tok, S), atol=1e-13)
