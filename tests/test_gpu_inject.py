"""GPU parity of dstill_inject_kv against oracle.drafter.Drafter.inject_rows.

Fusion H_t = RMSNorm(W_c feats) and injection K = rope(k_norm(W_k H_t)),
V = W_v H_t (DFlash review, Method / Inference) on the same features, row
sequence ids and positions.  Cache rows must match to 1e-5 relative (fp32) or,
in bf16, within 2 ulps plus 1/256 of the head vector's RMS (the fused state
H_t is itself rounded to bf16, and a rounding flip there moves a K/V value by
~1e-4 of the row scale);
rows with an invalid sequence id or position are not written; incremental
injection equals injecting everything at once (bit-exact).
"""

import numpy as np
import pytest
import torch

import block_diffusion_speculative_kv_amd as bd
from oracle.drafter import Drafter as OracleDrafter
from synth import configs, gen
from tests.helpers import assert_bf16_rows_close, assert_close_rel, device, to_np

pytestmark = pytest.mark.gpu


def _inject(cfg, n, cap, max_batch, seed_rows=0, invalid=()):
    dev = device()
    w = gen.weights(cfg, device=dev)
    dr = bd.Drafter(cfg, w)
    kv = dr.kv_cache(max_batch, cap)
    feats = gen.feats(cfg, n, device=dev)
    rng = np.random.default_rng(seed_rows)
    slots = rng.permutation(max_batch * cap)[:n]      # distinct cache rows
    seq, pos = slots // cap, slots % cap
    for i in invalid:
        seq[i] = -1 if i % 2 else max_batch
    seq_t = torch.from_numpy(seq.astype(np.int32)).to(dev)
    pos_t = torch.from_numpy(pos.astype(np.int32)).to(dev)
    ws = dr.workspace(max_inject_rows=n)
    dr.inject_kv(feats, seq_t, pos_t, kv, ws)
    torch.cuda.synchronize()
    return dev, w, dr, kv, feats, seq, pos, (seq_t, pos_t, ws)


def _check(cfg, w, kv, feats, seq, pos, rows):
    od = OracleDrafter(cfg, to_np(w))
    f_np = to_np(feats)[rows]
    ks, vs = od.inject_rows(f_np, pos[rows])
    for l in range(cfg["n_layers"]):
        K = to_np(kv.k[l])
        V = to_np(bd.KVCache.untile_v(kv.v[l]))
        gk = K[seq[rows], :, pos[rows]]          # [n, hkv, dh]
        gv = V[seq[rows], :, pos[rows]]
        if cfg["dtype"] == "f32":
            assert_close_rel(gk, ks[l], 1e-5, f"K layer {l}")
            assert_close_rel(gv, vs[l], 1e-5, f"V layer {l}")
        else:
            assert_bf16_rows_close(gk, ks[l], f"K layer {l}")
            assert_bf16_rows_close(gv, vs[l], f"V layer {l}")


def test_tiny_fp32():
    cfg = configs.get("tiny_fp32")
    dev, w, dr, kv, feats, seq, pos, _ = _inject(cfg, 128, 192, 1)
    _check(cfg, w, kv, feats, seq, pos, np.arange(128))


def test_small_bf16_with_skipped_rows():
    cfg = configs.small_bf16()
    n = 77
    invalid = (3, 10, 11)
    dev, w, dr, kv, feats, seq, pos, _ = _inject(cfg, n, 64, 3, invalid=invalid)
    ok = np.array([i not in invalid for i in range(n)])
    _check(cfg, w, kv, feats, seq, pos, np.nonzero(ok)[0])
    # every cache row not named by a valid input row is still zero
    written = set(zip(seq[ok].tolist(), pos[ok].tolist()))
    K = kv.k[0].float().cpu().numpy()
    for b in range(3):
        for p in range(64):
            if (b, p) not in written:
                assert not K[b, :, p].any()


def test_incremental_equals_all_at_once():
    cfg = configs.small_bf16()
    dev, w, dr, kv, feats, seq, pos, (seq_t, pos_t, ws) = _inject(cfg, 60, 64, 3)
    kv2 = dr.kv_cache(3, 64)
    for a, b in ((0, 7), (7, 31), (31, 60)):
        dr.inject_kv(feats[a:b].contiguous(), seq_t[a:b].contiguous(), pos_t[a:b].contiguous(),
                     kv2, ws)
    torch.cuda.synchronize()
    for l in range(cfg["n_layers"]):
        assert torch.equal(kv.k[l], kv2.k[l]) and torch.equal(kv.v[l], kv2.v[l])


def test_q8b_rows():
    cfg = configs.get("q8b_bs1_greedy")
    dev, w, dr, kv, feats, seq, pos, _ = _inject(cfg, 40, 4096, 1)
    _check(cfg, w, kv, feats, seq, pos, np.arange(40))


@pytest.mark.parametrize("n", [256, 259])
def test_q8b_256_rows(n):
    # 256 rows (the per-cycle injection at batch 32): the W_c and grouped K/V
    # products on the 128 x 256 tile; the K/V scatter pass takes four rows
    # per wave from 256 rows, and 259 leaves a partial group of three
    cfg = configs.get("q8b_bs1_greedy")
    dev, w, dr, kv, feats, seq, pos, _ = _inject(cfg, n, 4096, 1)
    _check(cfg, w, kv, feats, seq, pos, np.arange(n))


def test_many_rows_transposed_v_path():
    # 2500 rows (from 2048 rows the V rows are written by the row-tiled pass):
    # against the oracle, with skipped rows, and against the same rows
    # injected in chunks below that size (the per-row pass; the products then
    # run on other tiles and k-splits, so the two agree to bf16 rounding, not
    # bit for bit)
    cfg = configs.small_bf16()
    n = 2500
    invalid = (0, 999, 2047, 2048, 2499)
    dev, w, dr, kv, feats, seq, pos, (seq_t, pos_t, ws) = _inject(cfg, n, 1024, 3, invalid=invalid)
    ok = np.array([i not in invalid for i in range(n)])
    _check(cfg, w, kv, feats, seq, pos, np.nonzero(ok)[0][::7])
    kv2 = dr.kv_cache(3, 1024)
    for a, b in ((0, 1000), (1000, 2000), (2000, n)):
        dr.inject_kv(feats[a:b].contiguous(), seq_t[a:b].contiguous(), pos_t[a:b].contiguous(),
                     kv2, ws)
    torch.cuda.synchronize()
    rows = np.nonzero(ok)[0]
    for l in range(cfg["n_layers"]):
        for c1, c2, what in ((kv.k[l], kv2.k[l], "K"), (kv.v[l], kv2.v[l], "V")):
            a = c1.float().cpu().numpy() if what == "K" else \
                bd.KVCache.untile_v(c1).float().cpu().numpy()
            b = c2.float().cpu().numpy() if what == "K" else \
                bd.KVCache.untile_v(c2).float().cpu().numpy()
            assert_bf16_rows_close(a[seq[rows], :, pos[rows]], b[seq[rows], :, pos[rows]],
                                   f"{what} layer {l}: one call vs chunks")


def test_prefill_rows_vector_v_stores():
    # 2100 consecutive-position rows, as a prefill chunk gives them: from 2048
    # rows the V rows go through the row-tiled pass, which stores 8 keys at
    # once where 8 rows are 8 aligned consecutive positions of one sequence.
    # Sequence 0 takes rows 0..1002 (positions 0..1002), sequence 1 rows
    # 1003..2099 (positions 3..1099): the group of rows 1000..1007 straddles
    # the two, row 1500 is invalid (its group is stored element by element),
    # the other groups take the vector stores.  Against the oracle, the
    # untouched cache rows, and the same rows injected in chunks below 2048
    # rows (the per-row pass).
    cfg = configs.small_bf16()
    n, cap = 2100, 1152
    dev = device()
    w = gen.weights(cfg, device=dev)
    dr = bd.Drafter(cfg, w)
    feats = gen.feats(cfg, n, device=dev)
    seq = np.where(np.arange(n) < 1003, 0, 1)
    pos = np.where(seq == 0, np.arange(n), np.arange(n) - 1000)
    seq[1500] = -1
    seq_t = torch.from_numpy(seq.astype(np.int32)).to(dev)
    pos_t = torch.from_numpy(pos.astype(np.int32)).to(dev)
    ws = dr.workspace(max_inject_rows=n)
    kv = dr.kv_cache(2, cap)
    dr.inject_kv(feats, seq_t, pos_t, kv, ws)
    torch.cuda.synchronize()
    ok = seq >= 0
    rows = np.nonzero(ok)[0]
    _check(cfg, w, kv, feats, seq, pos, np.unique(np.concatenate(
        [rows[::9], rows[(rows >= 990) & (rows < 1020)], rows[(rows >= 1490) & (rows < 1512)],
         rows[-12:]])))
    # the slot of the invalid row (sequence 1, position 500) and the slots no
    # row names stay zero
    for l in range(cfg["n_layers"]):
        v = bd.KVCache.untile_v(kv.v[l]).float().cpu().numpy()
        assert not v[1, :, 500].any() and not v[0, :, 1003:].any() and not v[1, :, :3].any()
    kv2 = dr.kv_cache(2, cap)
    for a, b in ((0, 700), (700, 1400), (1400, n)):
        dr.inject_kv(feats[a:b].contiguous(), seq_t[a:b].contiguous(), pos_t[a:b].contiguous(),
                     kv2, ws)
    torch.cuda.synchronize()
    for l in range(cfg["n_layers"]):
        for c1, c2, what in ((kv.k[l], kv2.k[l], "K"), (kv.v[l], kv2.v[l], "V")):
            a = c1.float().cpu().numpy() if what == "K" else \
                bd.KVCache.untile_v(c1).float().cpu().numpy()
            b = c2.float().cpu().numpy() if what == "K" else \
                bd.KVCache.untile_v(c2).float().cpu().numpy()
            assert_bf16_rows_close(a[seq[rows], :, pos[rows]], b[seq[rows], :, pos[rows]],
                                   f"{what} layer {l}: one call vs chunks")


def test_q8b_three_layers_grouped_kv_off_the_192_tile():
    # 1001 rows, three 8B-shaped layers: the grouped K/V product (N = 3 x
    # 2048 = 6144, K = 4096) has the shape that takes 192-wide weight tiles,
    # but its 2048-row weight groups are not whole tiles of 192, so it runs on
    # the 256-wide tile under the split count planned for the 192-wide one;
    # the scatter pass ends on a single-row group
    cfg = configs.finish(dict(configs.WORKLOADS["q8b_bs1_greedy"], n_layers=3), "q8b_3layer")
    dev, w, dr, kv, feats, seq, pos, _ = _inject(cfg, 1001, 4096, 1)
    _check(cfg, w, kv, feats, seq, pos, np.arange(1001))
