"""Pins for the oracle's drafter (fusion, injection, block draft, LM head).

What fixes each part, other than the oracle itself:
* bfloat16 rounding: torch's float32 -> bfloat16 conversion (library routine).
* bfloat16 rounding points: an independent fp64 torch composition that rounds
  (frexp / round-half-even) at the stated points; leaving out any one point
  from the oracle breaks the agreement (mutation checks).
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


# -- bfloat16 rounding points -------------------------------------------------
#
# The oracle's bf16 mode rounds (round to nearest even) exactly where the
# library stores bfloat16: the fused state H_t, the cached K/V, the RMSNorm
# outputs fed to a projection, q and k after the rotary embedding, v, the
# attention output, the SiLU-times-up product and the final hidden state.
# An independent composition of torch routines in fp64 rounds at those points
# with a rounding of its own (frexp / round-half-even / ldexp, since torch's
# float64 -> bfloat16 conversion goes through float32 and so rounds twice);
# the two must agree to fp64 noise, and dropping any single rounding point
# from the oracle must break that agreement.

def _bf16_frexp(x):
    """Round to 8 significant bits, ties to even, through frexp / ldexp."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def test_frexp_rounding_is_bf16():
    rng = np.random.default_rng(12)
    x = rng.normal(0, 3, 200000).astype(np.float32)
    ties = (rng.integers(0x0080, 0x7F00, 1000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(_bf16_frexp(x.astype(np.float64)), want)
    # a float64 value just above a bfloat16 midpoint rounds up (one rounding)
    mid = 1.0 + 2.0 ** -8
    assert _bf16_frexp(np.array([mid + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert od.round_bf16(np.array([mid + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7


def _bf16_model(**kw):
    cfg = _tiny(dtype="bf16", **kw)
    w = _np(gen.weights(cfg))          # bf16 values, held as float64
    for lw in w["layers"]:
        lw["wqkv"] *= 8                # a power of two keeps them bf16 values
    return cfg, w


def _torch_inject_bf16(cfg, w, feats, pos, rb):
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    R = lambda t: T(rb(t.numpy()))
    qd, kvd, dh = cfg["q_dim"], cfg["kv_dim"], cfg["head_dim"]
    ht = R(F.rms_norm(F.linear(T(feats), T(w["w_fuse"])), (cfg["hidden"],),
                      T(w["g_fuse"]), cfg["rms_eps"]))
    ks, vs = [], []
    for lw in w["layers"]:
        k = F.linear(ht, T(lw["wqkv"])[qd:qd + kvd]).view(len(pos), -1, dh)
        k = _torch_rope(F.rms_norm(k, (dh,), T(lw["k_norm"]), cfg["rms_eps"]), list(pos),
                        cfg["rope_theta"])
        ks.append(rb(k.numpy()))
        vs.append(rb(F.linear(ht, T(lw["wqkv"])[qd + kvd:]).view(len(pos), -1, dh).numpy()))
    return ks, vs


def _torch_draft_bf16(cfg, w, ctx_k, ctx_v, tokens, S, rb):
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    R = lambda t: T(rb(t.numpy()))
    C, B = tokens.shape
    hq, hkv, dh, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["hidden"]
    eps = cfg["rms_eps"]
    h = F.embedding(torch.from_numpy(tokens.reshape(-1)).long(), T(w["embed"]))
    pos = [S + s for _ in range(C) for s in range(B)]
    for li, lw in enumerate(w["layers"]):
        u = R(F.rms_norm(h, (d,), T(lw["attn_norm"]), eps))
        q, k, v = F.linear(u, T(lw["wqkv"])).split([hq * dh, hkv * dh, hkv * dh], -1)
        q = R(_torch_rope(F.rms_norm(q.reshape(-1, hq, dh), (dh,), T(lw["q_norm"]), eps), pos,
                          cfg["rope_theta"]))
        k = R(_torch_rope(F.rms_norm(k.reshape(-1, hkv, dh), (dh,), T(lw["k_norm"]), eps), pos,
                          cfg["rope_theta"]))
        v = R(v.reshape(-1, hkv, dh))
        outs = []
        for c in range(C):
            sl = slice(c * B, (c + 1) * B)
            K = torch.cat([T(ctx_k[li])[:, :S], k[sl].transpose(0, 1)], 1)
            Vv = torch.cat([T(ctx_v[li])[:, :S], v[sl].transpose(0, 1)], 1)
            o = F.scaled_dot_product_attention(q[sl].transpose(0, 1)[None], K[None],
                                               Vv[None], enable_gqa=True)
            outs.append(o[0].transpose(0, 1).reshape(B, hq * dh))
        h = h + F.linear(R(torch.cat(outs, 0)), T(lw["wo"]))
        u = R(F.rms_norm(h, (d,), T(lw["mlp_norm"]), eps))
        g, up = F.linear(u, T(lw["w_gate_up"])).chunk(2, -1)
        h = h + F.linear(R(F.silu(g) * up), T(lw["w_down"]))
    return rb(F.rms_norm(h, (d,), T(w["g_final"]), eps).view(C, B, d).numpy())


class _SkipRound:
    """Oracle rounding that leaves out one rounding point: calls are counted
    per draft pass (seven per layer: attention-norm output, q, k, v, attention
    output, MLP-norm output, SiLU-times-up product; then the final state)."""

    def __init__(self, skip, per_layer=7):
        self.skip, self.per_layer, self.n = skip, per_layer, 0

    def __call__(self, x):
        i, self.n = self.n, self.n + 1
        if i % self.per_layer == self.skip or (self.skip == "final" and i == self.last):
            return np.asarray(x, dtype=np.float64)
        return od.round_bf16(x)


def _bf16_case(C=1, S=9):
    cfg, w = _bf16_model(n_copies=C)
    m = od.Drafter(cfg, w)
    rng = np.random.default_rng(13)
    n = max(S, 1)
    feats = _bf16_frexp(rng.normal(0, 1, (n, cfg["feat_dim"])))
    ks, vs = m.inject_rows(feats, np.arange(n))
    tokens = np.full((C, cfg["block"]), cfg["mask_token_id"])
    tokens[:, 0] = 7
    if C > 1:
        tokens[1:, 2] = rng.integers(0, 49, C - 1)
    return cfg, w, m, feats, ks, vs, tokens


@pytest.mark.parametrize("S,C", [(9, 1), (0, 1), (13, 3)])
def test_bf16_draft_rounding_points(S, C):
    cfg, w, m, feats, ks, vs, tokens = _bf16_case(C, S)
    ck = [k.transpose(1, 0, 2) for k in ks]
    cv = [v.transpose(1, 0, 2) for v in vs]
    got = m.draft(ck, cv, tokens, S)
    want = _torch_draft_bf16(cfg, w, ck, cv, tokens, S, _bf16_frexp)
    assert np.array_equal(_bf16_frexp(got), got)      # the final state is bf16
    assert np.allclose(got, want, rtol=0, atol=1e-9)
    # the f32-mode oracle on the same inputs differs: rounding happens at all
    m32 = od.Drafter(dict(cfg, dtype="f32"), w)
    assert np.abs(m32.draft(ck, cv, tokens, S) - want).max() > 1e-4


def test_bf16_injection_rounding_points():
    cfg, w, m, feats, ks, vs, _ = _bf16_case()
    pos = np.array([0, 5, 2, 9, 100, 3, 7, 1, 4])
    tk, tv = _torch_inject_bf16(cfg, w, feats, pos, _bf16_frexp)
    gk, gv = m.inject_rows(feats, pos)
    for li in range(cfg["n_layers"]):
        assert np.allclose(gk[li], tk[li], rtol=0, atol=1e-12)
        assert np.allclose(gv[li], tv[li], rtol=0, atol=1e-12)


@pytest.mark.parametrize("skip", [0, 1, 2])
def test_bf16_each_injection_rounding_point_is_needed(skip):
    """Mutation check: leaving out the round of H_t (call 0), of the cached K
    (call 1) or of the cached V (call 2) breaks the agreement."""
    cfg, w, m, feats, ks, vs, _ = _bf16_case()
    pos = np.array([0, 5, 2, 9, 100, 3, 7, 1, 4])
    tk, tv = _torch_inject_bf16(cfg, w, feats, pos, _bf16_frexp)
    calls = []

    def rb(x):
        calls.append(1)
        return np.asarray(x, np.float64) if len(calls) - 1 == skip else od.round_bf16(x)
    m.rb = rb
    gk, gv = m.inject_rows(feats, pos)
    assert len(calls) == 1 + 2 * cfg["n_layers"]
    assert max(np.abs(gk[0] - tk[0]).max(), np.abs(gv[0] - tv[0]).max()) > 1e-6


@pytest.mark.parametrize("skip", [0, 1, 2, 3, 4, 5, 6, "final"])
def test_bf16_each_rounding_point_is_needed(skip):
    """Mutation check: an oracle that leaves out any single rounding point no
    longer matches the independent composition."""
    S, C = 9, 1
    cfg, w, m, feats, ks, vs, tokens = _bf16_case(C, S)
    ck = [k.transpose(1, 0, 2) for k in ks]
    cv = [v.transpose(1, 0, 2) for v in vs]
    want = _torch_draft_bf16(cfg, w, ck, cv, tokens, S, _bf16_frexp)
    mut = _SkipRound(skip)
    mut.last = 7 * cfg["n_layers"]
    m.rb = mut
    got = m.draft(ck, cv, tokens, S)
    assert mut.n == 7 * cfg["n_layers"] + 1          # every point was visited
    assert np.abs(got - want).max() > 1e-6
