"""One draft + verify cycle over resident synthetic inputs.

A cycle is the four library calls in order (DFlash review, Method /
Inference and Preliminary; DStill, Inference):

  inject_kv       the target features of the n_new tokens verified last cycle
                  become context K/V in every draft layer
  block_draft     one pass over anchor + gamma masks (per copy)
  lm_head_argmax  shared head: greedy argmax, Gumbel-max sampling, or the
                  shared-Gumbel argmax of the multi-copy layout
  verify          greedy prefix match or rejection sampling; for the
                  multi-copy layout, SPOT's state-equality verification of
                  the drafted tree (root = copy 0)

With dloop_k = K > 0 (D-Loop, section 3.1 and 3.3) the head is followed by
the looped second pass: the K best prefix lengths of the first proposal are
re-drafted as K copies of the block (branch set-up, block_draft, head,
prefix/suffix merge), and the K branches are verified jointly, each against
its own synthetic target rows.

With refine_k = K > 0 (DStill, multi-step drafting) the draft and head run
K times per cycle on the evolving block state, each pass committing its most
confident masked positions (refine_commit); the endpoint is then verified.

The context cache is filled once by injecting every context row (prefill),
in chunks.  In steady state each cycle re-injects the n_new most recent
context positions of every sequence (the same slots every cycle), so every
timed cycle does identical work over identical shapes.  All tensors live on
the GPU before the first timed cycle; nothing is copied to or from the host
inside a cycle.
"""

from __future__ import annotations

import numpy as np
import torch

from synth import gen

from . import (Drafter, dloop_branches, dloop_merge, refine_commit, spot_verify, verify,
               verify_branches, verify_branches_workspace_bytes, verify_workspace_bytes)
from ._lib import HEAD_ARGMAX, HEAD_GUMBEL, HEAD_SHARED_GUMBEL, VERIFY_GREEDY, VERIFY_RS

_HEAD_MODE = {"argmax": HEAD_ARGMAX, "gumbel": HEAD_GUMBEL, "shared_gumbel": HEAD_SHARED_GUMBEL}


class Cycle:
    def __init__(self, cfg: dict, device="cuda", n_new: int = 8, prefill_chunk: int = 8192,
                 seed: int = 0):
        self.cfg = cfg
        self.dev = torch.device(device)
        bs, C, B, d = cfg["bs"], cfg["n_copies"], cfg["block"], cfg["hidden"]
        self.gamma = cfg["gamma"]
        self.ctx = list(cfg["ctx_lens"])
        self.max_ctx = max(self.ctx)
        self.n_new = max(1, min(n_new, min(self.ctx) if min(self.ctx) > 0 else 1))
        self.w = gen.weights(cfg, device=self.dev)
        self.dr = Drafter(cfg, self.w)
        self.kv = self.dr.kv_cache(bs, (self.max_ctx + B + 63) // 64 * 64)
        self.mode = _HEAD_MODE[cfg["lm_mode"]]
        self.verify_mode = {"greedy": VERIFY_GREEDY, "rs": VERIFY_RS}.get(cfg["verify"])
        self.spot = cfg["verify"] == "spot"
        self.yields = self.verify_mode is not None or self.spot  # tokens per cycle known
        self.T = float(cfg.get("temperature", 1.0))
        self.seed = seed
        # head rows: slots 1..gamma of every block, or all slots of every copy
        if self.mode == HEAD_SHARED_GUMBEL:
            self.rows, self.rows_per_seq, self.seq_stride, self.row0 = bs * C * B, B, B, 0
        else:
            self.rows, self.rows_per_seq, self.seq_stride, self.row0 = bs * C * self.gamma, \
                self.gamma, B, 1
        inj_rows = bs * self.n_new
        self.K = int(cfg.get("dloop_k", 0))
        self.rows2 = bs * self.K * self.gamma
        self.ws = self.dr.workspace(max_batch=bs, max_copies=max(C, self.K), max_ctx=self.max_ctx,
                                    max_inject_rows=max(inj_rows, min(prefill_chunk,
                                                                      sum(self.ctx) or 1)),
                                    max_head_rows=max(self.rows, self.rows2))
        self._prefill(prefill_chunk)
        # per-cycle inputs
        if self.spot:
            self.tokens, self.parent = gen.draft_tree(cfg, device=self.dev)
        else:
            self.tokens = gen.block_tokens(cfg, device=self.dev)
        self.ctx_len = torch.tensor(self.ctx, dtype=torch.int32, device=self.dev)
        self.feats = gen.feats(cfg, inj_rows, name="feats_cycle", device=self.dev)
        seq, pos = [], []
        for b, S in enumerate(self.ctx):
            for j in range(self.n_new):
                p = S - self.n_new + j
                seq.append(b if p >= 0 else -1)
                pos.append(max(p, 0))
        self.inj_seq = torch.tensor(seq, dtype=torch.int32, device=self.dev)
        self.inj_pos = torch.tensor(pos, dtype=torch.int32, device=self.dev)
        self.hidden = torch.empty((bs, C, B, d), dtype=self.dr.tdtype, device=self.dev)
        self.draft_flags = torch.zeros(bs, dtype=torch.int32, device=self.dev)
        r = self.rows
        self.ids = torch.empty(r, dtype=torch.int32, device=self.dev)
        self.zmax = torch.empty(r, dtype=torch.float32, device=self.dev)
        self.lse = torch.empty(r, dtype=torch.float32, device=self.dev)
        self.zsel = torch.empty(r, dtype=torch.float32, device=self.dev)
        self.gap = torch.empty(r, dtype=torch.float32, device=self.dev)
        self.logits = (torch.empty((r, cfg["vocab"]), dtype=torch.float32, device=self.dev)
                       if self.verify_mode == VERIFY_RS else None)
        if self.spot:
            i32 = torch.int32
            self.tau = torch.empty(bs, dtype=i32, device=self.dev)  # commits this round
            self.spot_slots = torch.empty((bs, C), dtype=i32, device=self.dev)
            self.spot_tokens = torch.empty((bs, C), dtype=i32, device=self.dev)
            self.spot_state = torch.empty(bs, dtype=i32, device=self.dev)
            self.vflags = torch.empty(bs, dtype=i32, device=self.dev)
        if self.verify_mode is not None:
            self.target = gen.target_logits(cfg, device=self.dev)
            self.out_tokens = torch.empty((bs, self.gamma + 1), dtype=torch.int32,
                                          device=self.dev)
            self.tau = torch.empty(bs, dtype=torch.int32, device=self.dev)
            self.vflags = torch.empty(bs, dtype=torch.int32, device=self.dev)
            self.vws = torch.empty(verify_workspace_bytes(bs, self.gamma, cfg["vocab"]),
                                   dtype=torch.uint8, device=self.dev)
        self.RK = int(cfg.get("refine_k", 0))
        if self.RK:
            self.rtok0 = self.tokens.view(bs, B).clone()
            self.rtok = self.rtok0.clone()
            self.rkap0 = torch.full((bs, B), -1, dtype=torch.int32, device=self.dev)
            self.rkap0[:, 0] = 0
            self.rkap = self.rkap0.clone()
            self.rids = torch.empty((bs, self.gamma), dtype=torch.int32, device=self.dev)
        if self.K:
            K, g, i32 = self.K, self.gamma, torch.int32
            self.anchor = self.tokens[:, 0, 0].contiguous()
            self.blocks = torch.empty((bs, K, B), dtype=i32, device=self.dev)
            self.prefix_len = torch.empty((bs, K), dtype=i32, device=self.dev)
            self.hidden2 = torch.empty((bs, K, B, d), dtype=self.dr.tdtype, device=self.dev)
            self.ids2 = torch.empty(self.rows2, dtype=i32, device=self.dev)
            self.proposal = torch.empty((bs, K, g), dtype=i32, device=self.dev)
            self.branch = torch.empty(bs, dtype=i32, device=self.dev)
            self.target_br = gen.normal((bs, K, g + 1, cfg["vocab"]), cfg["target_logit_std"],
                                        seed=cfg["seed"], name="target_branches", device=self.dev)
            self.vws_br = torch.empty(verify_branches_workspace_bytes(bs, K, g, cfg["vocab"]),
                                      dtype=torch.uint8, device=self.dev)
        torch.cuda.synchronize(self.dev)

    def prefill_chunk(self, chunk: int = 8192):
        """The first prefill chunk (features, sequence ids, positions), for
        timing an injection at prefill size; injecting it again rewrites the
        same cache rows with the same values."""
        rows = [(b, p) for b, S in enumerate(self.ctx) for p in range(S)][:chunk]
        f = gen.feats(self.cfg, len(rows), name="feats_prefill0", device=self.dev)
        seq = torch.tensor([b for b, _ in rows], dtype=torch.int32, device=self.dev)
        pos = torch.tensor([p for _, p in rows], dtype=torch.int32, device=self.dev)
        return f, seq, pos

    def _prefill(self, chunk):
        rows = [(b, p) for b, S in enumerate(self.ctx) for p in range(S)]
        for i in range(0, len(rows), chunk):
            part = rows[i:i + chunk]
            f = gen.feats(self.cfg, len(part), name=f"feats_prefill{i}", device=self.dev)
            seq = torch.tensor([b for b, _ in part], dtype=torch.int32, device=self.dev)
            pos = torch.tensor([p for _, p in part], dtype=torch.int32, device=self.dev)
            self.dr.inject_kv(f, seq, pos, self.kv, self.ws)
        torch.cuda.synchronize(self.dev)

    # -- the four calls -------------------------------------------------------
    def inject(self):
        self.dr.inject_kv(self.feats, self.inj_seq, self.inj_pos, self.kv, self.ws)

    def draft(self):
        self.dr.block_draft(self.tokens, self.ctx_len, self.max_ctx, self.kv, self.hidden, self.ws,
                            flags=self.draft_flags)

    def head(self, cycle: int):
        hv = self.hidden.view(-1, self.cfg["hidden"])[self.row0:]
        self.dr.lm_head_argmax(hv, self.rows, self.rows_per_seq, self.seq_stride, self.ids,
                               self.ws, mode=self.mode, temperature=self.T, seed=self.seed,
                               cycle=cycle, zmax=self.zmax, lse=self.lse, zsel=self.zsel,
                               gap=self.gap, logits=self.logits)

    def refine(self, cycle: int):
        """K drafter passes over the evolving block state, each followed by
        the head and the commit of its most confident positions."""
        bs, g, B = self.cfg["bs"], self.gamma, self.cfg["block"]
        self.rtok.copy_(self.rtok0)
        self.rkap.copy_(self.rkap0)
        for t in range(1, self.RK + 1):
            self.dr.block_draft(self.rtok.view(bs, 1, B), self.ctx_len, self.max_ctx, self.kv,
                                self.hidden, self.ws, flags=self.draft_flags)
            self.head(cycle)
            refine_commit(self.ids.view(bs, g), self.zmax.view(bs, g), self.lse.view(bs, g), t,
                          self.RK, self.rtok, self.rkap)
        self.rids.copy_(self.rtok[:, 1:])

    def loop(self, cycle: int):
        """D-Loop second pass: branches, K-copy draft, head, merge."""
        if not self.K:
            return
        bs, g, B, d = self.cfg["bs"], self.gamma, self.cfg["block"], self.cfg["hidden"]
        dloop_branches(self.anchor, self.ids.view(bs, g), self.zmax.view(bs, g),
                       self.lse.view(bs, g), self.K, self.cfg["mask_token_id"], self.blocks,
                       self.prefix_len)
        self.dr.block_draft(self.blocks, self.ctx_len, self.max_ctx, self.kv, self.hidden2,
                            self.ws)
        self.dr.lm_head_argmax(self.hidden2.view(-1, d)[1:], self.rows2, g, B, self.ids2,
                               self.ws, mode=HEAD_ARGMAX, cycle=cycle)
        dloop_merge(self.ids.view(bs, g), self.ids2.view(bs, self.K, g), self.prefix_len,
                    self.proposal)

    def verify(self, cycle: int):
        bs = self.cfg["bs"]
        if self.spot:
            C, B = self.cfg["n_copies"], self.cfg["block"]
            sh = (bs, C, B)
            spot_verify(self.tokens, self.parent, self.ids.view(sh), self.zmax.view(sh),
                        self.lse.view(sh), self.cfg["mask_token_id"], self.tau, self.spot_slots,
                        self.spot_tokens, self.spot_state, self.vflags, temperature=self.T,
                        gap=self.gap.view(sh))
            return
        if self.verify_mode is None:
            return
        if self.K:
            verify_branches(self.proposal, self.target_br, self.out_tokens, self.tau,
                            self.branch, self.vflags, self.vws_br)
            return
        ids = self.rids if self.RK else self.ids.view(bs, self.gamma)
        verify(self.verify_mode, ids, self.target, self.out_tokens,
               self.tau, self.vflags, self.vws, temperature=self.T, seed=self.seed, cycle=cycle,
               draft_lse=self.lse.view(bs, self.gamma) if self.logits is not None else None,
               draft_logits=(self.logits.view(bs, self.gamma, -1)
                             if self.logits is not None else None))

    # -- planted acceptance (harness only) ------------------------------------
    def can_plant(self) -> bool:
        return (self.verify_mode is not None and not (self.K or self.RK or self.spot)
                and self.cfg["n_copies"] == 1)

    def plant_draw(self, cycle: int, alpha: float) -> np.ndarray:
        """Accepted-prefix lengths k in [0, gamma] per sequence: each draft
        position is accepted with probability alpha independently until the
        first rejection (P(k) = alpha^k (1 - alpha) for k < gamma, alpha^gamma
        at k = gamma), so E[tau] = 1 + sum_{j=1..gamma} alpha^j; drawn on the
        host from the cycle's own stream of numbers."""
        rng = np.random.default_rng([int(self.seed), 4, int(cycle)])
        acc = rng.random((self.cfg["bs"], self.gamma)) < alpha
        return np.where(acc.all(axis=1), self.gamma, np.argmin(acc, axis=1))

    def _plant(self, k: np.ndarray):
        """Makes target row j of sequence b favour the drafted token y_{j+1}
        for j < k_b (greedy: it is the row's argmax; rejection sampling: p(y)
        = 1, so the ratio p/q >= 1 accepts) and give it no mass at j = k_b
        (greedy mismatch; p(y) = 0 rejects), so tau_b = k_b + 1.  Returns
        what is needed to undo it."""
        bs, g = self.cfg["bs"], self.gamma
        y = self.ids.view(bs, g).long()
        kk = torch.as_tensor(k, device=self.dev).view(bs, 1)
        j = torch.arange(g, device=self.dev).view(1, g)
        bi = torch.arange(bs, device=self.dev).view(bs, 1).expand(bs, g)
        ji = j.expand(bs, g)
        old = self.target[bi, ji, y].clone()
        new = torch.where(j < kk, torch.full_like(old, 1e4),
                          torch.where(j == kk, torch.full_like(old, -1e4), old))
        self.target[bi, ji, y] = new
        return bi, ji, y, old

    def step(self, cycle: int = 0, plant_k: np.ndarray = None):
        """One cycle.  plant_k (plain one-pass cycles with verification only)
        plants those accepted-prefix lengths into the target rows between the
        head and the verification and restores the rows afterwards."""
        self.inject()
        if self.RK:
            self.refine(cycle)
        else:
            self.draft()
            self.head(cycle)
            self.loop(cycle)
        undo = self._plant(plant_k) if plant_k is not None else None
        self.verify(cycle)
        if undo is not None:
            bi, ji, y, old = undo
            self.target[bi, ji, y] = old
