"""Plain float64 definition of the drafter: feature fusion, KV injection,
one-pass block draft and the shared LM head.  Test infrastructure only.

Page references (cited by page title and section):

* DFlash review, "Method / Inference", feature fusion and KV injection
  equations: H_t = RMSNorm(W_c [H^l1; ...; H^lnf]); for draft layer i,
  Q_i = W_i^Q H_d, K_i = [W_i^K H_t; W_i^K H_d], V_i = [W_i^V H_t; W_i^V H_d];
  the injected context K/V persist across drafting iterations.
* DStill, "Setup and notation": block x_1 = (a, [MASK], ..., [MASK]) of B
  positions; the drafter attends bidirectionally inside the block and to the
  target context strictly before the anchor; one distribution per masked
  position.  "Experimental Setup": drafters reuse the target's frozen
  embedding and LM head.
* DStill, appendix drafter table: Qwen3-style transformer layers.  Readings
  (the pages give no more): pre-norm RMSNorm, per-head q/k RMSNorm, rotary
  position embedding with rotate-half pairing (i, i + dh/2), grouped-query
  attention with scale 1/sqrt(dh) and no mask among context + block keys,
  SwiGLU MLP, residual adds, a final RMSNorm, no biases.
* SPOT, "Method" (multi-copy layout): with several copies of a block, a copy's
  queries see the shared prefix and that copy's own block keys only.

bfloat16 rounding (round to nearest even) is applied only where the library
stores bfloat16; all other arithmetic is float64.
"""

from __future__ import annotations

import numpy as np


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float64.  Values are assumed finite and in the normal float32 range."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64)


def _ident(x):
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, g, eps):
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope(x, pos, theta):
    """Rotary embedding of x [n, h, dh] at integer positions pos [n]: the pair
    (i, i + dh/2) is rotated by pos * theta^(-2i/dh)."""
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    half = dh // 2
    inv = float(theta) ** (-np.arange(half, dtype=np.float64) * 2.0 / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def softmax(s, axis=-1):
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def logsumexp(s, axis=-1):
    m = np.max(s, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=axis, keepdims=True))
            ).squeeze(axis)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


class Drafter:
    """Drafter weights (numpy arrays, any float dtype) plus the workload
    geometry.  Weight names and layouts are those of ``synth.gen.weights``:
    [out, in] row-major; wqkv rows are W^Q, W^K, W^V; w_gate_up rows are
    gate then up."""

    def __init__(self, cfg: dict, w: dict):
        self.cfg = cfg
        self.w = w
        self.rb = round_bf16 if cfg["dtype"] == "bf16" else _ident
        self.eps = float(cfg["rms_eps"])
        self.theta = float(cfg["rope_theta"])
        self.hq, self.hkv = cfg["n_q_heads"], cfg["n_kv_heads"]
        self.dh = cfg["head_dim"]
        self.qd, self.kvd = self.hq * self.dh, self.hkv * self.dh

    # -- feature fusion and KV injection ---------------------------------
    def fuse(self, feats):
        """H_t = RMSNorm(W_c . feats) with gain g_fuse, one row per token."""
        x = _f64(feats) @ _f64(self.w["w_fuse"]).T
        return self.rb(rms_norm(x, self.w["g_fuse"], self.eps))

    def _head_norm(self, x, g):
        if not self.cfg["qk_norm"]:
            return x
        return rms_norm(x, g, self.eps)

    def inject_rows(self, feats, pos):
        """Context K/V for every draft layer from target features of tokens at
        positions pos: K = rope(knorm(W^K H_t)), V = W^V H_t.
        Returns lists over layers of K, V arrays [n, h_kv, dh]."""
        pos = np.asarray(pos)
        ht = self.fuse(feats)
        n = ht.shape[0]
        ks, vs = [], []
        for lw in self.w["layers"]:
            wkv = _f64(lw["wqkv"][self.qd:self.qd + 2 * self.kvd])
            kv = ht @ wkv.T
            k = kv[:, :self.kvd].reshape(n, self.hkv, self.dh)
            v = kv[:, self.kvd:].reshape(n, self.hkv, self.dh)
            k = rope(self._head_norm(k, lw["k_norm"]), pos, self.theta)
            ks.append(self.rb(k))
            vs.append(self.rb(v))
        return ks, vs

    # -- one-pass block draft -------------------------------------------
    def draft(self, ctx_k, ctx_v, tokens, S, trace=None):
        """One forward pass over a block of one sequence.

        ctx_k, ctx_v: lists over layers of [h_kv, >=S, dh] injected context
        K/V (rows 0..S-1 are used).  tokens: [C, B] block token ids (copy c,
        slot s; slot 0 is the anchor), the block sits at positions S..S+B-1.
        Returns the final-normed hidden state [C, B, d]."""
        tokens = np.asarray(tokens)
        C, B = tokens.shape
        n = C * B
        rb = self.rb
        h = _f64(self.w["embed"][tokens.reshape(-1)])
        pos = np.tile(S + np.arange(B), C)
        group = self.hq // self.hkv
        scale = 1.0 / np.sqrt(self.dh)
        for li, lw in enumerate(self.w["layers"]):
            u = rb(rms_norm(h, lw["attn_norm"], self.eps))
            qkv = u @ _f64(lw["wqkv"]).T
            q = qkv[:, :self.qd].reshape(n, self.hq, self.dh)
            k = qkv[:, self.qd:self.qd + self.kvd].reshape(n, self.hkv, self.dh)
            v = qkv[:, self.qd + self.kvd:].reshape(n, self.hkv, self.dh)
            q = rb(rope(self._head_norm(q, lw["q_norm"]), pos, self.theta))
            k = rb(rope(self._head_norm(k, lw["k_norm"]), pos, self.theta))
            v = rb(v)
            q = q.reshape(C, B, self.hq, self.dh)
            k = k.reshape(C, B, self.hkv, self.dh)
            v = v.reshape(C, B, self.hkv, self.dh)
            out = np.empty((C, B, self.hq, self.dh))
            # sliding window (DStill appendix drafter table, SWA layers): the
            # block sees the last W context positions; full layers see all
            W = int(self.cfg.get("swa_window", 0))
            full = (int(self.cfg.get("full_attn_mask", 0)) >> li) & 1
            lo = max(0, S - W) if W > 0 and not full else 0
            ck = _f64(ctx_k[li])[:, lo:S]
            cv = _f64(ctx_v[li])[:, lo:S]
            for c in range(C):
                for j in range(self.hq):
                    g = j // group
                    keys = np.concatenate([ck[g], k[c, :, g]], axis=0)
                    vals = np.concatenate([cv[g], v[c, :, g]], axis=0)
                    p = softmax(q[c, :, j] @ keys.T * scale, axis=-1)
                    out[c, :, j] = p @ vals
            attn = rb(out.reshape(n, self.qd))
            h = h + attn @ _f64(lw["wo"]).T
            u = rb(rms_norm(h, lw["mlp_norm"], self.eps))
            gu = u @ _f64(lw["w_gate_up"]).T
            m = self.cfg["mlp"]
            act = rb(silu(gu[:, :m]) * gu[:, m:])
            h = h + act @ _f64(lw["w_down"]).T
            if trace is not None:
                trace.append(dict(q=q, k=k, v=v, attn=attn, h=h.copy()))
        hf = rb(rms_norm(h, self.w["g_final"], self.eps))
        return hf.reshape(C, B, -1)


def lm_head(w_lm, hidden, temperature=1.0, gumbel=None, keep_logits=False):
    """Shared LM head over rows of final hidden states.

    z = hidden . W_lm^T.  The selected id is argmax z (greedy: top-1 per
    position) or, with Gumbel noise g [rows, V], argmax (z / T + g), which is
    a draw from softmax(z / T) (Gumbel-max).  Ties go to the lowest id.
    Returns ids, zmax = max z, lse = log sum exp(z / T), zsel = z[id] and gap =
    winner minus runner-up of the scored quantity."""
    z = _f64(hidden) @ _f64(w_lm).T
    T = float(temperature)
    score = z if gumbel is None else z / T + _f64(gumbel)
    ids = np.argmax(score, axis=-1)
    rows = np.arange(z.shape[0])
    top = score[rows, ids]
    masked = score.copy()
    masked[rows, ids] = -np.inf
    gap = top - np.max(masked, axis=-1)
    out = dict(ids=ids.astype(np.int64), zmax=np.max(z, axis=-1),
               lse=logsumexp(z / T, axis=-1), zsel=z[rows, ids], gap=gap)
    if keep_logits:
        out["logits"] = z
    return out
