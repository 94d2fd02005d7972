"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

Every tensor is drawn from its own torch generator whose seed is a stable hash
of (workload seed, tensor name), so a tensor is reproducible on its own and the
same call on the same device always returns the same values.  Large tensors are
drawn directly on the GPU; the oracle receives host copies of exactly those
tensors.  Distributions (standard deviations, not variances):

  weights        N(0, 0.02)          RMSNorm gains   1 + N(0, 0.1)
  embedding      N(0, 0.02)          target features N(0, 1)
  target logits  N(0, std)           synthetic KV    N(0, 1)

This module holds no arithmetic of the method.
"""

from __future__ import annotations

import zlib

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def _seed(seed: int, name: str) -> int:
    return (int(seed) * 1000003 + zlib.crc32(name.encode())) & ((1 << 62) - 1)


def _gen(device, seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, name))
    return g


def normal(shape, std, mean=0.0, *, seed, name, device="cpu",
           dtype=torch.float32):
    g = _gen(device, seed, name)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)


def integers(shape, lo, hi, *, seed, name, device="cpu"):
    """Integers uniform in [lo, hi) as int32."""
    g = _gen(device, seed, name)
    return torch.randint(lo, hi, shape, generator=g, device=device,
                         dtype=torch.int64).to(torch.int32)


def weights(cfg: dict, device="cpu", seed=None) -> dict:
    """Drafter weights in the workload dtype, [out, in] row-major.

    Layer tensors: attn_norm [d], wqkv [(hq+2hkv)*dh, d] (rows: W^Q, W^K,
    W^V), q_norm [dh], k_norm [dh], wo [d, hq*dh], mlp_norm [d],
    w_gate_up [2*mlp, d] (rows: gate then up), w_down [d, mlp].
    """
    s = cfg["seed"] if seed is None else seed
    dt = torch_dtype(cfg["dtype"])
    d, dh, V = cfg["hidden"], cfg["head_dim"], cfg["vocab"]
    qd, kvd, F, m = cfg["q_dim"], cfg["kv_dim"], cfg["feat_dim"], cfg["mlp"]

    def w(shape, name):
        return normal(shape, 0.02, seed=s, name=name, device=device, dtype=dt)

    def gain(n, name):
        return normal((n,), 0.1, 1.0, seed=s, name=name, device=device,
                      dtype=dt)

    out = dict(
        embed=w((V, d), "embed"),
        lm_head=w((V, d), "lm_head"),
        w_fuse=w((d, F), "w_fuse"),
        g_fuse=gain(d, "g_fuse"),
        g_final=gain(d, "g_final"),
        layers=[],
    )
    for i in range(cfg["n_layers"]):
        p = f"layer{i}."
        out["layers"].append(dict(
            attn_norm=gain(d, p + "attn_norm"),
            wqkv=w((qd + 2 * kvd, d), p + "wqkv"),
            q_norm=gain(dh, p + "q_norm"),
            k_norm=gain(dh, p + "k_norm"),
            wo=w((d, qd), p + "wo"),
            mlp_norm=gain(d, p + "mlp_norm"),
            w_gate_up=w((2 * m, d), p + "w_gate_up"),
            w_down=w((d, m), p + "w_down"),
        ))
    return out


def feats(cfg: dict, n: int, name="feats", device="cpu", seed=None):
    s = cfg["seed"] if seed is None else seed
    return normal((n, cfg["feat_dim"]), 1.0, seed=s, name=name, device=device,
                  dtype=torch_dtype(cfg["dtype"]))


def target_logits(cfg: dict, device="cpu", name="target_logits", seed=None):
    """[bs, gamma+1, V] target logits, N(0, target_logit_std)."""
    s = cfg["seed"] if seed is None else seed
    return normal((cfg["bs"], cfg["gamma"] + 1, cfg["vocab"]),
                  cfg["target_logit_std"], seed=s, name=name, device=device,
                  dtype=torch_dtype(cfg["target_dtype"]))


def draft_logits(cfg: dict, device="cpu", name="draft_logits", seed=None,
                 std=None):
    s = cfg["seed"] if seed is None else seed
    std = cfg["target_logit_std"] if std is None else std
    return normal((cfg["bs"], cfg["gamma"], cfg["vocab"]), std, seed=s,
                  name=name, device=device, dtype=torch.float32)


def block_tokens(cfg: dict, device="cpu", seed=None):
    """[bs, n_copies, B] int32: anchor at slot 0, mask id elsewhere.  Copies
    after the first reveal a random subset of slots with random tokens (the
    multi-copy layout); the first copy is always the root state."""
    s = cfg["seed"] if seed is None else seed
    bs, C, B, V = cfg["bs"], cfg["n_copies"], cfg["block"], cfg["vocab"]
    mask = cfg["mask_token_id"]
    anchor = integers((bs,), 0, V - 1, seed=s, name="anchor", device=device)
    tok = torch.full((bs, C, B), mask, dtype=torch.int32, device=device)
    tok[:, :, 0] = anchor[:, None]
    if C > 1:
        reveal = integers((bs, C - 1, B - 1), 0, 2, seed=s, name="reveal",
                          device=device).bool()
        fill = integers((bs, C - 1, B - 1), 0, V - 1, seed=s, name="fill",
                        device=device)
        sub = tok[:, 1:, 1:]
        tok[:, 1:, 1:] = torch.where(reveal, fill, sub)
    return tok


def draft_tree(cfg: dict, device="cpu", seed=None):
    """A root block state and n_copies - 1 drafted states for the multi-copy
    layout: tokens [bs, n_copies, B] int32 (state 0 = anchor + masks) and
    parent [bs, n_copies] int32 (-1 for the root).  Draft j extends a random
    earlier state by one random token at one of its masked slots."""
    s = cfg["seed"] if seed is None else seed
    bs, C, B, V = cfg["bs"], cfg["n_copies"], cfg["block"], cfg["vocab"]
    mask = cfg["mask_token_id"]
    g = _gen("cpu", s, "draft_tree")
    tok = torch.full((bs, C, B), mask, dtype=torch.int32)
    par = torch.full((bs, C), -1, dtype=torch.int32)
    for b in range(bs):
        tok[b, 0, 0] = int(torch.randint(0, V - 1, (1,), generator=g))
        for j in range(1, C):
            p = int(torch.randint(0, j, (1,), generator=g))
            st = tok[b, p].clone()
            m = (st == mask).nonzero().flatten()
            if m.numel():
                k = int(m[int(torch.randint(0, m.numel(), (1,), generator=g))])
                st[k] = int(torch.randint(0, V - 1, (1,), generator=g))
            tok[b, j] = st
            par[b, j] = p
    return tok.to(device), par.to(device)


def kv_cache(cfg: dict, cap: int, device="cpu", seed=None, name="kv"):
    """Synthetic per-layer K/V caches [bs, h_kv, cap, dh], N(0, 1), in the
    workload dtype (stands in for an injected context when a test exercises
    the draft step on its own)."""
    s = cfg["seed"] if seed is None else seed
    dt = torch_dtype(cfg["dtype"])
    shape = (cfg["bs"], cfg["n_kv_heads"], cap, cfg["head_dim"])
    ks, vs = [], []
    for i in range(cfg["n_layers"]):
        ks.append(normal(shape, 1.0, seed=s, name=f"{name}.k{i}", device=device,
                         dtype=dt))
        vs.append(normal(shape, 1.0, seed=s, name=f"{name}.v{i}", device=device,
                         dtype=dt))
    return ks, vs


def hidden_rows(cfg: dict, rows: int, device="cpu", seed=None, name="hidden"):
    s = cfg["seed"] if seed is None else seed
    return normal((rows, cfg["hidden"]), 1.0, seed=s, name=name, device=device,
                  dtype=torch_dtype(cfg["dtype"]))
