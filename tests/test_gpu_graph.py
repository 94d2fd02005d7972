"""One whole cycle (injection, block draft or refinement, LM head, D-Loop
pass, verification) captured into a HIP graph through torch's CUDAGraph and
replayed.  None of the library's calls allocates, synchronises or records a
memset, so the captured cycle must reproduce the eager one bit for bit.

Each replay starts from outputs overwritten with a sentinel and follows an
eager cycle with a different cycle number (other random draws under Gumbel
drafting and rejection sampling, so other values in the same buffers); the
eager cycle that follows each replay must still give its own results.
Variants: greedy with argmax drafting, rejection sampling with Gumbel
drafting and bf16 target rows, the D-Loop second pass, iterative refinement
and tree (spot) verification of several copies, all on the reduced bf16
drafter.
"""

import pytest
import torch

from block_diffusion_speculative_kv_amd.cycle import Cycle
from synth import configs
from tests.helpers import device

pytestmark = pytest.mark.gpu

_OUT = ("hidden", "ids", "zmax", "lse", "zsel", "gap", "logits", "out_tokens", "tau", "vflags",
        "draft_flags", "hidden2", "ids2", "blocks", "prefix_len", "proposal", "branch", "rtok",
        "rkap", "rids", "spot_slots", "spot_tokens", "spot_state")

_CASES = {
    "greedy": dict(verify="greedy", lm_mode="argmax", target_dtype="f32"),
    "rs_gumbel": dict(verify="rs", lm_mode="gumbel", target_dtype="bf16",
                      target_logit_std=3.0),
    "dloop": dict(bs=2, ctx=[37, 300], verify="greedy", lm_mode="argmax", dloop_k=3),
    "refine": dict(bs=2, ctx=[37, 300], verify="greedy", lm_mode="argmax", refine_k=3),
    "spot": dict(bs=2, ctx=[37, 300], n_copies=3, verify="spot", lm_mode="shared_gumbel"),
}


def _bufs(cyc):
    return {n: getattr(cyc, n) for n in _OUT if getattr(cyc, n, None) is not None}


def _smear(cyc):
    """Overwrites every output with a byte pattern no cycle writes whole."""
    for t in _bufs(cyc).values():
        t.view(torch.uint8).fill_(0xA5)


def _snap(cyc):
    return {n: t.view(torch.uint8).clone() for n, t in _bufs(cyc).items()}


def _same(got, ref, what):
    for n in ref:
        assert torch.equal(got[n], ref[n]), f"{what}: {n} differs"


@pytest.mark.parametrize("case", list(_CASES))
def test_cycle_graph_replay(case):
    cfg = configs.small_bf16(**_CASES[case])
    cyc = Cycle(cfg, device=device(), n_new=4)
    _smear(cyc)
    cyc.step(cycle=5)
    torch.cuda.synchronize()
    ref5 = _snap(cyc)
    _smear(cyc)
    cyc.step(cycle=6)
    torch.cuda.synchronize()
    ref6 = _snap(cyc)
    if case in ("rs_gumbel", "spot"):  # the cycle number reaches the draws
        assert any(not torch.equal(ref5[n], ref6[n]) for n in ref5)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cyc.step(cycle=5)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cyc.step(cycle=5)
    torch.cuda.synchronize()

    for r in range(3):
        _smear(cyc)
        g.replay()
        torch.cuda.synchronize()
        _same(_snap(cyc), ref5, f"replay {r}")
        _smear(cyc)
        cyc.step(cycle=6)
        torch.cuda.synchronize()
        _same(_snap(cyc), ref6, f"eager cycle after replay {r}")
    del g
