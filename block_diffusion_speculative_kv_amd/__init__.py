"""One-pass block-diffusion drafting with lossless verification on MI355X.

Thin Python binding over the C ABI of libdstill.so (include/dstill.h).  The
four calls keep the ABI's names: ``Drafter.inject_kv``, ``Drafter.block_draft``,
``Drafter.lm_head_argmax`` and the model-independent ``verify``.  Tensors are
torch tensors on the GPU; torch provides device memory and the stream, the
library does every step of the computation.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (BF16, F32, FLAG_BAD_INPUT, FLAG_CTX_CLAMPED, FLAG_NEAR_THRESHOLD,
                   FLAG_NEAR_TIE_SAMPLE, FLAG_NEAR_TIE_TARGET, FLAG_ZERO_RESIDUAL, HEAD_ARGMAX,
                   HEAD_GUMBEL, HEAD_SHARED_GUMBEL, NEAR, NOALLOC_SCRATCH_BYTES, VERIFY_GREEDY,
                   VERIFY_RS, DstillError)

__all__ = [
    "Drafter", "verify", "verify_noalloc", "verify_workspace_bytes", "DstillError", "F32",
    "BF16", "HEAD_ARGMAX", "HEAD_GUMBEL", "HEAD_SHARED_GUMBEL", "VERIFY_GREEDY", "VERIFY_RS", "FLAG_NEAR_TIE_TARGET",
    "FLAG_NEAR_THRESHOLD", "FLAG_NEAR_TIE_SAMPLE", "FLAG_ZERO_RESIDUAL", "FLAG_BAD_INPUT",
    "FLAG_CTX_CLAMPED", "NEAR",
    "dloop_branches", "dloop_merge", "verify_branches", "verify_branches_workspace_bytes",
    "spot_verify", "refine_commit",
]

_DT = {"f32": F32, "bf16": BF16}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_check(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors passed to the library must be contiguous CUDA tensors")


class Drafter:
    """A drafter handle over caller-owned weights.

    cfg: workload dict (see synth.configs) with the model geometry.
    weights: dict of GPU tensors in the layout of synth.gen.weights.
    """

    def __init__(self, cfg: dict, weights: dict):
        self.lib = _lib.load()
        self.cfg = cfg
        self.dtype = _DT[cfg["dtype"]]
        self.tdtype = _TORCH_DT[self.dtype]
        self._w = weights  # keep tensors alive
        c = _lib.Config(
            n_layers=cfg["n_layers"], hidden=cfg["hidden"], n_q_heads=cfg["n_q_heads"],
            n_kv_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"], mlp=cfg["mlp"],
            vocab=cfg["vocab"], n_feat_layers=cfg["n_feat_layers"],
            target_hidden=cfg["target_hidden"], max_block=cfg["block"],
            mask_token_id=cfg["mask_token_id"], qk_norm=int(cfg["qk_norm"]), dtype=self.dtype,
            rms_eps=float(cfg["rms_eps"]), rope_theta=float(cfg["rope_theta"]),
            swa_window=int(cfg.get("swa_window", 0)),
            full_attn_mask=int(cfg.get("full_attn_mask", 0)))
        self._cfg_c = c
        L = len(weights["layers"])
        self._layers = (_lib.LayerWeights * L)()
        for i, lw in enumerate(weights["layers"]):
            _dev_check(*lw.values())
            for name in ("attn_norm", "wqkv", "q_norm", "k_norm", "wo", "mlp_norm",
                         "w_gate_up", "w_down"):
                setattr(self._layers[i], name, lw[name].data_ptr())
        _dev_check(weights["embed"], weights["lm_head"], weights["w_fuse"],
                   weights["g_fuse"], weights["g_final"])
        w = _lib.Weights(embed=weights["embed"].data_ptr(), lm_head=weights["lm_head"].data_ptr(),
                         w_fuse=weights["w_fuse"].data_ptr(), g_fuse=weights["g_fuse"].data_ptr(),
                         g_final=weights["g_final"].data_ptr(), layers=self._layers)
        h = ctypes.c_void_p()
        _lib.check(self.lib.dstill_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)),
                   "dstill_create")
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self.lib.dstill_destroy(h)
            self.handle = None

    # -- memory helpers ------------------------------------------------------
    def kv_cache(self, max_batch: int, cap: int, device="cuda"):
        """Allocate (zeroed) per-layer caches: K [max_batch, h_kv, cap, dh] and
        V in 64-position tiles [max_batch, h_kv, cap/64, dh, 64] (cap a
        multiple of 64)."""
        n = ctypes.c_size_t()
        _lib.check(self.lib.dstill_kv_bytes(ctypes.byref(self._cfg_c), max_batch, cap,
                                            ctypes.byref(n)), "dstill_kv_bytes")
        hk, dh = self.cfg["n_kv_heads"], self.cfg["head_dim"]
        ks = [torch.zeros((max_batch, hk, cap, dh), dtype=self.tdtype, device=device)
              for _ in range(self.cfg["n_layers"])]
        vs = [torch.zeros((max_batch, hk, cap // 64, dh, 64), dtype=self.tdtype, device=device)
              for _ in range(self.cfg["n_layers"])]
        assert ks[0].numel() * ks[0].element_size() == n.value
        return KVCache(ks, vs)

    def workspace_bytes(self, max_batch=1, max_copies=1, max_ctx=1, max_inject_rows=0,
                        max_head_rows=0) -> int:
        lim = _lib.Limits(max_batch=max_batch, max_copies=max_copies, max_ctx=max_ctx,
                          max_inject_rows=max_inject_rows, max_head_rows=max_head_rows)
        n = ctypes.c_size_t()
        _lib.check(self.lib.dstill_workspace_bytes(self.handle, ctypes.byref(lim), ctypes.byref(n)),
                   "dstill_workspace_bytes")
        return n.value

    def workspace(self, device="cuda", **limits):
        return torch.empty(max(1, self.workspace_bytes(**limits)), dtype=torch.uint8, device=device)

    # -- the three model calls ----------------------------------------------
    def inject_kv(self, feats, seq_id, pos, kv: "KVCache", ws, stream=None):
        _dev_check(feats, seq_id, pos, ws)
        n = feats.shape[0] if feats.dim() == 2 else 0
        _lib.check(self.lib.dstill_inject_kv(self.handle, _ptr(feats), _ptr(seq_id), _ptr(pos), n,
                                             ctypes.byref(kv.c), _ptr(ws), ws.numel(),
                                             _stream(stream)), "dstill_inject_kv")

    def block_draft(self, block_tokens, ctx_len, max_ctx: int, kv: "KVCache", hidden_out, ws,
                    flags=None, stream=None):
        """block_tokens [bs, n_copies, B] int32; ctx_len [bs] int32; hidden_out
        [bs, n_copies, B, hidden] in the drafter dtype."""
        _dev_check(block_tokens, ctx_len, hidden_out, ws, flags)
        bs, C, B = block_tokens.shape
        _lib.check(self.lib.dstill_block_draft(self.handle, _ptr(block_tokens), _ptr(ctx_len), bs,
                                               B, C, int(max_ctx), ctypes.byref(kv.c),
                                               _ptr(hidden_out), _ptr(flags), _ptr(ws), ws.numel(),
                                               _stream(stream)), "dstill_block_draft")

    def lm_head_argmax(self, hidden, rows: int, rows_per_seq: int, seq_stride: int, ids, ws, *,
                       mode=HEAD_ARGMAX, temperature=1.0, seed=0, cycle=0, zmax=None, lse=None,
                       zsel=None, gap=None, logits=None, stream=None):
        """hidden: tensor whose data pointer is row 0 (see the header's row
        addressing); outputs [rows] (logits [rows, vocab] fp32)."""
        _dev_check(ids, ws, zmax, lse, zsel, gap, logits)
        if not hidden.is_cuda:
            raise ValueError("hidden must be a CUDA tensor")
        s = _lib.Sample(mode=mode, temperature=float(temperature), seed=int(seed), cycle=int(cycle))
        _lib.check(self.lib.dstill_lm_head_argmax(
            self.handle, _ptr(hidden), rows, rows_per_seq, seq_stride, ctypes.byref(s), _ptr(ids),
            _ptr(zmax), _ptr(lse), _ptr(zsel), _ptr(gap), _ptr(logits), _ptr(ws), ws.numel(),
            _stream(stream)), "dstill_lm_head_argmax")


class KVCache:
    """Per-layer K [max_batch, h_kv, cap, dh] and tiled V [max_batch, h_kv,
    cap/64, dh, 64] cache tensors plus the C view the library reads."""

    @staticmethod
    def tile_v(v_rows):
        """[b, h, cap, dh] position-major V -> the library's tiled layout."""
        b, h, cap, dh = v_rows.shape
        return v_rows.view(b, h, cap // 64, 64, dh).transpose(-1, -2).contiguous()

    @staticmethod
    def untile_v(v_tiled):
        """The library's tiled V -> [b, h, cap, dh]."""
        b, h, nt, dh, _ = v_tiled.shape
        return v_tiled.transpose(-1, -2).reshape(b, h, nt * 64, dh)

    def __init__(self, ks, vs):
        self.k, self.v = ks, vs
        L = len(ks)
        self._kp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in ks])
        self._vp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in vs])
        self.c = _lib.KV(k=self._kp, v=self._vp, max_batch=ks[0].shape[0], cap=ks[0].shape[2])


def verify_workspace_bytes(bs: int, gamma: int, vocab: int) -> int:
    lib = _lib.load()
    n = ctypes.c_size_t()
    _lib.check(lib.dstill_verify_workspace_bytes(bs, gamma, vocab, ctypes.byref(n)),
               "dstill_verify_workspace_bytes")
    return n.value


def verify(mode: int, draft_ids, target_logits, out_tokens, out_tau, out_flags, ws, *,
           temperature=1.0, seed=0, cycle=0, draft_lse=None, draft_logits=None, stream=None):
    """draft_ids [bs, gamma] int32; target_logits [bs, gamma+1, V] fp32/bf16;
    outputs tokens [bs, gamma+1] int32, tau [bs] int32, flags [bs] int32."""
    lib = _lib.load()
    _dev_check(draft_ids, target_logits, out_tokens, out_tau, out_flags, ws, draft_lse,
               draft_logits)
    bs, g1, V = target_logits.shape
    tdt = BF16 if target_logits.dtype == torch.bfloat16 else F32
    if target_logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("target logits must be fp32 or bf16")
    _lib.check(lib.dstill_verify(mode, bs, g1 - 1, V, float(temperature), int(seed), int(cycle),
                                 _ptr(draft_ids), _ptr(draft_lse), _ptr(draft_logits),
                                 _ptr(target_logits), tdt, _ptr(out_tokens), _ptr(out_tau),
                                 _ptr(out_flags), _ptr(ws), ws.numel(), _stream(stream)),
               "dstill_verify")


def verify_noalloc(mode: int, draft_ids, target_logits, out_tokens, out_tau, out_flags, *,
                   temperature=1.0, seed=0, cycle=0, draft_lse=None, draft_logits=None,
                   stream=None):
    """verify() without a workspace argument: the library's fixed per-device
    scratch (NOALLOC_SCRATCH_BYTES) serves as workspace; nothing is allocated.
    Calls that overlap on one device race on that scratch."""
    lib = _lib.load()
    _dev_check(draft_ids, target_logits, out_tokens, out_tau, out_flags, draft_lse, draft_logits)
    bs, g1, V = target_logits.shape
    tdt = BF16 if target_logits.dtype == torch.bfloat16 else F32
    if target_logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("target logits must be fp32 or bf16")
    _lib.check(lib.dstill_verify_noalloc(mode, bs, g1 - 1, V, float(temperature), int(seed),
                                         int(cycle), _ptr(draft_ids), _ptr(draft_lse),
                                         _ptr(draft_logits), _ptr(target_logits), tdt,
                                         _ptr(out_tokens), _ptr(out_tau), _ptr(out_flags),
                                         _stream(stream)), "dstill_verify_noalloc")


# ---- D-Loop second pass ------------------------------------------------------
def dloop_branches(anchor, ids, zmax, lse, K: int, mask_id: int, block_tokens, prefix_len,
                   score=None, stream=None):
    """anchor [bs], first-pass ids / zmax / lse [bs, gamma] -> block_tokens
    [bs, K, gamma+1] int32, prefix_len [bs, K] int32, score [bs, K] fp64."""
    lib = _lib.load()
    _dev_check(anchor, ids, zmax, lse, block_tokens, prefix_len, score)
    bs, g = ids.shape
    _lib.check(lib.dstill_dloop_branches(bs, g, K, _ptr(anchor), _ptr(ids), _ptr(zmax), _ptr(lse),
                                         int(mask_id), _ptr(block_tokens), _ptr(prefix_len),
                                         _ptr(score), _stream(stream)), "dstill_dloop_branches")


def dloop_merge(first_ids, second_ids, prefix_len, out_ids, stream=None):
    """first_ids [bs, gamma], second_ids [bs, K, gamma], prefix_len [bs, K]
    -> out_ids [bs, K, gamma] (int32)."""
    lib = _lib.load()
    _dev_check(first_ids, second_ids, prefix_len, out_ids)
    bs, K, g = second_ids.shape
    _lib.check(lib.dstill_dloop_merge(bs, g, K, _ptr(first_ids), _ptr(second_ids),
                                      _ptr(prefix_len), _ptr(out_ids), _stream(stream)),
               "dstill_dloop_merge")


def verify_branches_workspace_bytes(bs: int, K: int, gamma: int, vocab: int) -> int:
    lib = _lib.load()
    n = ctypes.c_size_t()
    _lib.check(lib.dstill_verify_branches_workspace_bytes(bs, K, gamma, vocab, ctypes.byref(n)),
               "dstill_verify_branches_workspace_bytes")
    return n.value


def verify_branches(draft_ids, target_logits, out_tokens, out_tau, out_branch, out_flags, ws,
                    stream=None):
    """draft_ids [bs, K, gamma] int32; target_logits [bs, K, gamma+1, V]
    fp32/bf16 -> tokens [bs, gamma+1], tau [bs], branch [bs], flags [bs]."""
    lib = _lib.load()
    _dev_check(draft_ids, target_logits, out_tokens, out_tau, out_branch, out_flags, ws)
    bs, K, g1, V = target_logits.shape
    if target_logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("target logits must be fp32 or bf16")
    tdt = BF16 if target_logits.dtype == torch.bfloat16 else F32
    _lib.check(lib.dstill_verify_branches(bs, K, g1 - 1, V, _ptr(draft_ids), _ptr(target_logits),
                                          tdt, _ptr(out_tokens), _ptr(out_tau), _ptr(out_branch),
                                          _ptr(out_flags), _ptr(ws), ws.numel(), _stream(stream)),
               "dstill_verify_branches")


# ---- SPOT state-equality verification -------------------------------------------
def spot_verify(states, parent, ids, zmax, lse, mask_id: int, out_n, out_slots, out_tokens,
                out_state, out_flags, *, temperature=1.0, gap=None, stream=None):
    """states / ids / zmax / lse / gap [bs, n_states, L]; parent [bs, n_states]
    -> out_n [bs], out_slots / out_tokens [bs, n_states], out_state [bs],
    out_flags [bs]."""
    lib = _lib.load()
    _dev_check(states, parent, ids, zmax, lse, gap, out_n, out_slots, out_tokens, out_state,
               out_flags)
    bs, n, L = states.shape
    _lib.check(lib.dstill_spot_verify(bs, n, L, int(mask_id), float(temperature), _ptr(states),
                                      _ptr(parent), _ptr(ids), _ptr(zmax), _ptr(lse), _ptr(gap),
                                      _ptr(out_n), _ptr(out_slots), _ptr(out_tokens),
                                      _ptr(out_state), _ptr(out_flags), _stream(stream)),
               "dstill_spot_verify")


# ---- multi-step refinement ----------------------------------------------------------
def refine_commit(ids, zmax, lse, t: int, K: int, tokens, kappa, stream=None):
    """ids / zmax / lse [bs, block-1] of pass t of K; tokens, kappa [bs, block]
    int32, updated in place."""
    lib = _lib.load()
    _dev_check(ids, zmax, lse, tokens, kappa)
    bs, B = tokens.shape
    _lib.check(lib.dstill_refine_commit(bs, B, int(t), int(K), _ptr(ids), _ptr(zmax), _ptr(lse),
                                        _ptr(tokens), _ptr(kappa), _stream(stream)),
               "dstill_refine_commit")
