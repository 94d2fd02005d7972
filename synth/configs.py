"""Workload shapes for the one-pass block-diffusion draft + verify path.

Each workload is a plain dict.  Shapes follow the pages: a DFlash-style drafter
of a few Qwen3-style layers conditioned on fused target features (DFlash review,
"Method / Inference"), block size 16 = one anchor + 15 masked positions (DStill,
"Setup and notation"; DFlash review, "Experiments / Setup"), five target feature
layers (same setup paragraph), and the SPOT multi-copy verify layout of D draft
copies appended behind a cached prefix (SPOT, "Method").

This module holds no arithmetic of the method: only sizes and seeds.
"""

from __future__ import annotations

import copy

# Common Qwen3-8B-sized drafter geometry (hidden 4096, 32 query / 8 KV heads of
# 128, SwiGLU MLP 12288, vocabulary 151936, 5 layers, 5 fused target layers).
_Q8B = dict(
    n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
    mlp=12288, vocab=151936, n_feat_layers=5, target_hidden=4096,
    gamma=15, dtype="bf16", rms_eps=1e-6, rope_theta=1e6, qk_norm=1,
)

WORKLOADS = {
    # Tiny fp32 drafter, greedy verify, batch 1.
    "tiny_fp32": dict(
        n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
        mlp=1024, vocab=1024, n_feat_layers=3, target_hidden=256,
        gamma=7, dtype="f32", rms_eps=1e-6, rope_theta=1e6, qk_norm=1,
        bs=1, ctx=[128], n_copies=1, verify="greedy", lm_mode="argmax",
        temperature=1.0, target_logit_std=2.0, target_dtype="f32", seed=0,
    ),
    # 8B-shaped drafter, batch 1, context 4096, greedy.
    "q8b_bs1_greedy": dict(
        _Q8B, bs=1, ctx=[4096], n_copies=1, verify="greedy",
        lm_mode="argmax", temperature=1.0, target_logit_std=2.0,
        target_dtype="f32", seed=0,
    ),
    # 8B-shaped drafter, batch 32, ragged contexts U[1024, 8192], T=1
    # rejection sampling with sampled (Gumbel-max) drafting, bf16 target logits.
    "q8b_bs32_rs": dict(
        _Q8B, bs=32, ctx="uniform:1024:8192:0", n_copies=1, verify="rs",
        lm_mode="gumbel", temperature=1.0, target_logit_std=3.0,
        target_dtype="bf16", seed=0,
    ),
    # Long context: batch 4, context 32768, greedy.
    "q8b_bs4_long": dict(
        _Q8B, bs=4, ctx=[32768] * 4, n_copies=1, verify="greedy",
        lm_mode="argmax", temperature=1.0, target_logit_std=2.0,
        target_dtype="f32", seed=0,
    ),
    # Multi-copy verify shape: root block + 8 drafted states of 16 positions
    # behind a 4096-token prefix, copy-local attention, shared-Gumbel argmax,
    # state-equality verification of the draft tree.
    "q8b_multicopy": dict(
        _Q8B, bs=1, ctx=[4096], n_copies=9, verify="spot",
        lm_mode="shared_gumbel", temperature=1.0, target_logit_std=2.0,
        target_dtype="f32", seed=0,
    ),
    # D-Loop looped second pass (K = 4 branches) on the bs-1 greedy workload:
    # first pass, top-4 prefix branches re-drafted as 4 copies of the block,
    # joint greedy verification of the 4 branches.
    "q8b_dloop_k4": dict(
        _Q8B, bs=1, ctx=[4096], n_copies=1, verify="greedy",
        lm_mode="argmax", temperature=1.0, target_logit_std=2.0,
        target_dtype="f32", seed=0, dloop_k=4,
    ),
    # DStill multi-step refinement (the teacher rollout): 8 drafter passes per
    # block on the bs-1 greedy workload, each committing its most confident
    # positions, then greedy verification of the endpoint.
    "q8b_refine_k8": dict(
        _Q8B, bs=1, ctx=[4096], n_copies=1, verify="greedy",
        lm_mode="argmax", temperature=1.0, target_logit_std=2.0,
        target_dtype="f32", seed=0, refine_k=8,
    ),
    # Sliding-window drafter (SWA 2048 in every layer, as on the Gemma and
    # Nemotron drafters) on the long-context shape: batch 4, context 32768.
    "q8b_swa_long": dict(
        _Q8B, bs=4, ctx=[32768] * 4, n_copies=1, verify="greedy",
        lm_mode="argmax", temperature=1.0, target_logit_std=2.0,
        target_dtype="f32", seed=0, swa_window=2048,
    ),
}

# Order used when a workload is referred to by index (0 = the tiny case).
ORDER = ["tiny_fp32", "q8b_bs1_greedy", "q8b_bs32_rs", "q8b_bs4_long",
         "q8b_multicopy"]


def get(name: str, **overrides) -> dict:
    """Return a copy of a workload dict with derived fields filled in."""
    cfg = copy.deepcopy(WORKLOADS[name])
    cfg.update(overrides)
    return finish(cfg, name)


def finish(cfg: dict, name: str = "custom") -> dict:
    cfg = dict(cfg)
    cfg.setdefault("name", name)
    cfg["block"] = cfg["gamma"] + 1
    cfg.setdefault("mask_token_id", cfg["vocab"] - 1)
    cfg["feat_dim"] = cfg["n_feat_layers"] * cfg["target_hidden"]
    cfg["q_dim"] = cfg["n_q_heads"] * cfg["head_dim"]
    cfg["kv_dim"] = cfg["n_kv_heads"] * cfg["head_dim"]
    cfg["ctx_lens"] = context_lengths(cfg)
    return cfg


def context_lengths(cfg: dict) -> list[int]:
    """Per-sequence context lengths S_b (the anchor sits at position S_b).

    A spec "uniform:lo:hi:seed" draws integers in [lo, hi] inclusive from
    numpy's default_rng(seed), as the ragged batch of the bs=32 workload.
    """
    ctx = cfg["ctx"]
    if isinstance(ctx, str):
        import numpy as np
        kind, lo, hi, seed = ctx.split(":")
        assert kind == "uniform"
        rng = np.random.default_rng(int(seed))
        return [int(x) for x in rng.integers(int(lo), int(hi) + 1, cfg["bs"])]
    assert len(ctx) == cfg["bs"]
    return [int(x) for x in ctx]


def small_bf16(**overrides) -> dict:
    """A reduced bf16 drafter that still spans several kernel tiles and has
    ragged tails (vocab and contexts not multiples of any tile size); the
    oracle finishes it in seconds."""
    base = dict(
        n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
        mlp=1408, vocab=5003, n_feat_layers=3, target_hidden=384,
        gamma=15, dtype="bf16", rms_eps=1e-6, rope_theta=1e6, qk_norm=1,
        bs=3, ctx=[37, 300, 1029], n_copies=1, verify="greedy",
        lm_mode="argmax", temperature=1.0, target_logit_std=2.0,
        target_dtype="f32", seed=1,
    )
    base.update(overrides)
    return finish(base, "small_bf16")
