"""GPU parity of dstill_lm_head_argmax against oracle.drafter.lm_head.

Both sides get the same hidden rows and the same LM-head weight (bf16 or
fp32, drawn on the GPU by synth.gen).  The oracle computes the full logits in
fp64 and takes the argmax / log-sum-exp / Gumbel-max over them; the kernel
never stores logits unless asked and reduces them on the fly.  Ids must agree
bit-exactly wherever neither side's top-2 score gap is below 1e-5 (those rows
are counted, recorded and bounded).  In fp32 the statistics and stored logits
must agree to 1e-5 * max(1, |oracle|); in bf16 (fp32 accumulation of bf16
products over d = 4096 terms) to the recursive-summation bound
2.5e-4 * sum_k |h_k w_k|, ~1e-4 absolute for these inputs.

Shapes: the tiny fp32 workload (V 1024, d 256, gamma 7 rows), ragged bf16
cases (V 5003, d 512, rows in blocks of 15 with a stride of 16) at 11, 30,
37, 45, 100 and 300 rows (the streaming kernel with 1, 2 and 3 row tiles,
the 128 x 160 tile, two row blocks of the largest tile), the 64 x 32 and
64 x 64 tiles at depth 576 (not a multiple of the streaming stage), and the
full 8B-shaped head (V 151936, d 4096) at the row counts of the greedy bs-1
(15 rows, argmax), bs-4 (60 rows), bs-32 rejection-sampling (480 rows,
Gumbel, logits stored) and multi-copy (144 rows, shared Gumbel) workloads,
every row checked.
"""

import numpy as np
import pytest
import torch

import block_diffusion_speculative_kv_amd as bd
from oracle import philox
from oracle.drafter import lm_head as oracle_head
from synth import configs, gen
from tests.helpers import compare_ids, device, to_np

pytestmark = pytest.mark.gpu

_TD = {"f32": torch.float32, "bf16": torch.bfloat16}


class _HeadOnly:
    """A drafter handle whose other weights are tiny placeholders: only the
    LM head is exercised."""

    def __init__(self, V, d, dtype, seed):
        self.cfg = configs.finish(dict(
            n_layers=1, hidden=d, n_q_heads=1, n_kv_heads=1, head_dim=64, mlp=32, vocab=V,
            n_feat_layers=1, target_hidden=32, gamma=15, dtype=dtype, rms_eps=1e-6,
            rope_theta=1e6, qk_norm=1, bs=1, ctx=[0], n_copies=1, seed=seed))
        dev = device()
        td = _TD[dtype]
        self.w_lm = gen.normal((V, d), 0.02, seed=seed, name="lm_head", device=dev, dtype=td)
        z = lambda *s: torch.zeros(*s, dtype=td, device=dev)
        layer = dict(attn_norm=z(d), wqkv=z(3 * 64, d), q_norm=z(64), k_norm=z(64), wo=z(d, 64),
                     mlp_norm=z(d), w_gate_up=z(64, d), w_down=z(d, 32))
        self.w = dict(embed=z(V, d), lm_head=self.w_lm, w_fuse=z(d, 32), g_fuse=z(d),
                      g_final=z(d), layers=[layer])
        self.dr = bd.Drafter(self.cfg, self.w)


def _gumbel_rows(mode, seed, cycle, seqs, slots, V):
    purpose = philox.PURPOSE_SHARED if mode == bd.HEAD_SHARED_GUMBEL else philox.PURPOSE_DRAFT
    seqs = np.zeros_like(seqs) if mode == bd.HEAD_SHARED_GUMBEL else np.asarray(seqs)
    j = np.arange(V, dtype=np.uint64)[None, :]
    out = []
    for a in range(0, len(seqs), 16):
        s = seqs[a:a + 16, None].astype(np.uint64)
        p = np.asarray(slots)[a:a + 16, None].astype(np.uint64)
        out.append(philox.gumbel(seed, purpose, s, p, cycle, j))
    return np.concatenate(out)


def _run_case(V, d, dtype, rows, rows_per_seq, seq_stride, mode, T=1.0, keep_logits=False,
              sample=None, seed=5, cycle=3):
    h = _HeadOnly(V, d, dtype, seed)
    dev = device()
    nseq = (rows + rows_per_seq - 1) // rows_per_seq
    hid_all = gen.normal((nseq * seq_stride, d), 1.0, seed=seed, name="hidden", device=dev,
                         dtype=_TD[dtype])
    ids = torch.empty(rows, dtype=torch.int32, device=dev)
    outs = {k: torch.empty(rows, dtype=torch.float32, device=dev)
            for k in ("zmax", "lse", "zsel", "gap")}
    logits = torch.empty((rows, V), dtype=torch.float32, device=dev) if keep_logits else None
    ws = h.dr.workspace(max_head_rows=rows)
    h.dr.lm_head_argmax(hid_all, rows, rows_per_seq, seq_stride, ids, ws, mode=mode,
                        temperature=T, seed=seed, cycle=cycle, logits=logits, **outs)
    torch.cuda.synchronize()
    # rows checked against the oracle
    r_idx = np.arange(rows) if sample is None else np.unique(
        np.linspace(0, rows - 1, sample).astype(int))
    seqs, slots = r_idx // rows_per_seq, r_idx % rows_per_seq
    hrows = seqs * seq_stride + slots
    hid_np = to_np(hid_all)[hrows]
    W = to_np(h.w_lm)
    g = None if mode == bd.HEAD_ARGMAX else _gumbel_rows(mode, seed, cycle, seqs, slots, V)
    ref = oracle_head(W, hid_np, temperature=T, gumbel=g, keep_logits=True)
    if dtype == "f32":
        bound = 1e-5 * np.maximum(1.0, np.abs(ref["logits"]))   # 1e-5 relative
    else:
        bound = 2.5e-4 * (np.abs(hid_np) @ np.abs(W).T)        # fp32 accumulation bound
    zb = bound.max(-1)
    got = {k: v.cpu().numpy().astype(np.float64)[r_idx] for k, v in outs.items()}
    gids = ids.cpu().numpy()[r_idx]
    excl = (ref["gap"] < 1e-5) | (got["gap"] < 1e-5)
    n = compare_ids(gids, ref["ids"], excl, f"lm_head V{V} mode{mode}")
    ok = ~excl
    if dtype == "f32":
        rel = lambda a, b: np.abs(a - b) / np.maximum(1.0, np.abs(b))
        assert rel(got["zmax"], ref["zmax"]).max() <= 1e-5
        assert rel(got["zsel"][ok], ref["zsel"][ok]).max(initial=0) <= 1e-5
        assert rel(got["lse"], ref["lse"]).max() <= 1e-5
        assert np.all(np.abs(got["gap"][ok] - ref["gap"][ok]) <= 2 * zb[ok] / min(T, 1.0))
    else:
        assert np.all(np.abs(got["zmax"] - ref["zmax"]) <= zb)
        assert np.all(np.abs(got["zsel"][ok] - ref["zsel"][ok]) <= zb[ok])
        # lse of z/T: each term's error is bounded by the logit bound / T
        assert np.all(np.abs(got["lse"] - ref["lse"]) <= zb / T + 1e-6 * np.abs(ref["lse"]))
        assert np.all(np.abs(got["gap"][ok] - ref["gap"][ok]) <= 2 * zb[ok] / min(T, 1.0) + 1e-5)
    if keep_logits:
        L = logits.cpu().numpy().astype(np.float64)[r_idx]
        assert np.all(np.abs(L - ref["logits"]) <= bound)
    return n, ids.cpu().numpy(), r_idx


def test_tiny_fp32_argmax():
    n, _, _ = _run_case(1024, 256, "f32", 7, 7, 8, bd.HEAD_ARGMAX, keep_logits=True)
    assert n == 0


def test_ragged_bf16_gumbel_strided_rows():
    _run_case(5003, 512, "bf16", 37, 15, 16, bd.HEAD_GUMBEL, T=0.8, keep_logits=True)


def test_ragged_bf16_argmax():
    _run_case(5003, 512, "bf16", 45, 15, 16, bd.HEAD_ARGMAX)


def test_ragged_bf16_gumbel_up_to_32_rows():
    # 17..32 rows: the streaming kernel with two row tiles
    _run_case(5003, 512, "bf16", 30, 15, 16, bd.HEAD_GUMBEL, keep_logits=True)


def test_ragged_bf16_stream_up_to_16_rows():
    # <= 16 rows: the streaming kernel with one row tile, partial last vocabulary block
    _run_case(5003, 512, "bf16", 11, 11, 16, bd.HEAD_GUMBEL, T=1.3, keep_logits=True)


@pytest.mark.parametrize("rows,mode", [(30, bd.HEAD_GUMBEL), (60, bd.HEAD_ARGMAX)])
def test_ragged_bf16_tiles_off_the_streaming_depth(rows, mode):
    # depth 576 is a whole number of 64-deep tile stages but not of 128-deep
    # streaming stages: the 64 x 32 and 64 x 64 tiles of the tile engine
    _run_case(5003, 576, "bf16", rows, 15, 16, mode, keep_logits=True)


@pytest.mark.parametrize("rows", [80, 100, 150])
def test_ragged_bf16_gumbel_up_to_160_rows(rows):
    # 65..160 rows: the streaming kernel with 64-deep stages and 6, 8 or 10
    # row tiles (the last one ragged), partial last vocabulary block
    _run_case(5003, 512, "bf16", rows, 15, 16, bd.HEAD_GUMBEL, T=0.9, keep_logits=True)


def test_ragged_bf16_argmax_two_row_blocks():
    # > 160 rows: the 256 x 256 tile over two row blocks (the second partial)
    _run_case(5003, 512, "bf16", 300, 15, 16, bd.HEAD_ARGMAX, keep_logits=True)


def test_q8b_bs4_rows(parity_record):
    # 60 rows (4 sequences x 15 slots): the streaming kernel with four row
    # tiles (three-stage ring) at full vocabulary
    n, _, _ = _run_case(151936, 4096, "bf16", 60, 15, 16, bd.HEAD_ARGMAX)
    parity_record(rows=60, near_tie_rows=n)
    assert n <= 1


def test_q8b_greedy_bs1_rows(parity_record):
    n, _, _ = _run_case(151936, 4096, "bf16", 15, 15, 16, bd.HEAD_ARGMAX)
    parity_record(rows=15, near_tie_rows=n)
    assert n <= 1


def test_q8b_bs32_gumbel_with_logits(parity_record):
    # every one of the 480 rows: ids, statistics and the stored logits
    n, _, _ = _run_case(151936, 4096, "bf16", 480, 15, 16, bd.HEAD_GUMBEL, keep_logits=True)
    parity_record(rows=480, near_tie_rows=n)
    assert n <= 1


def test_q8b_multicopy_shared_gumbel(parity_record):
    n, ids, r_idx = _run_case(151936, 4096, "bf16", 144, 16, 16, bd.HEAD_SHARED_GUMBEL)
    parity_record(rows=144, near_tie_rows=n)
    assert n <= 1


def test_shared_gumbel_identical_rows_agree():
    # copies of one hidden row at the same slot share the noise: same draw
    h = _HeadOnly(5003, 512, "bf16", 1)
    dev = device()
    row = gen.normal((1, 512), 1.0, seed=1, name="hidden", device=dev, dtype=torch.bfloat16)
    hid = row.repeat(4 * 16, 1).contiguous()
    ids = torch.empty(64, dtype=torch.int32, device=dev)
    ws = h.dr.workspace(max_head_rows=64)
    h.dr.lm_head_argmax(hid, 64, 16, 16, ids, ws, mode=bd.HEAD_SHARED_GUMBEL, seed=3, cycle=1)
    got = ids.cpu().numpy().reshape(4, 16)
    assert np.all(got == got[0])           # every copy agrees slot by slot
    assert len(set(got[0].tolist())) > 1   # slots draw different noise
