"""dstill_verify_noalloc (the verification call that allocates nothing and
uses the library's fixed per-device scratch) against dstill_verify with a
caller workspace, through the C ABI.

Both calls get the same inputs; tokens, tau and flags must be identical (the
two run the same kernels on the same inputs, only the workspace differs).
Two calls in a row on the shared scratch, the second with a smaller shape, so
stale records of the first call cannot leak into the second; both verify
modes (greedy at the bs-1 shape, rejection sampling at the bs-32 shape with
the full 8B-shaped vocabulary); the rejection of a shape beyond the scratch.
"""

import numpy as np
import pytest
import torch

import block_diffusion_speculative_kv_amd as bd
from oracle.drafter import logsumexp
from synth import gen
from tests.helpers import device, to_np

pytestmark = pytest.mark.gpu


def _outs(bs, g1, dev):
    return (torch.full((bs, g1), -7, dtype=torch.int32, device=dev),
            torch.zeros(bs, dtype=torch.int32, device=dev),
            torch.full((bs,), -1, dtype=torch.int32, device=dev))


def _inputs(mode, bs, gamma, V, seed):
    dev = device()
    cfg = dict(bs=bs, gamma=gamma, vocab=V, target_logit_std=3.0,
               target_dtype="bf16" if mode == bd.VERIFY_RS else "f32", seed=seed)
    zt = gen.target_logits(cfg, device=dev)
    zd = gen.draft_logits(cfg, device=dev) if mode == bd.VERIFY_RS else None
    rng = np.random.default_rng(seed)
    if mode == bd.VERIFY_RS:
        y = torch.from_numpy(np.argmax(to_np(zd), -1).astype(np.int32)).to(dev)
        lse = torch.from_numpy(logsumexp(to_np(zd), -1).astype(np.float32)).to(dev)
    else:
        t = np.argmax(to_np(zt), -1)[:, :gamma]
        y_np = rng.integers(0, V, (bs, gamma))
        k = rng.integers(0, gamma + 1, bs)
        for b in range(bs):
            y_np[b, :k[b]] = t[b, :k[b]]
        y = torch.from_numpy(y_np.astype(np.int32)).to(dev)
        lse = None
    return zt, zd, y, lse


def _both(mode, zt, zd, y, lse, seed, cycle):
    bs, g1, V = zt.shape
    dev = zt.device
    ref = _outs(bs, g1, dev)
    ws = torch.empty(bd.verify_workspace_bytes(bs, g1 - 1, V), dtype=torch.uint8, device=dev)
    bd.verify(mode, y, zt, *ref, ws, seed=seed, cycle=cycle, draft_lse=lse, draft_logits=zd)
    got = _outs(bs, g1, dev)
    bd.verify_noalloc(mode, y, zt, *got, seed=seed, cycle=cycle, draft_lse=lse, draft_logits=zd)
    torch.cuda.synchronize()
    for a, b, name in zip(got, ref, ("tokens", "tau", "flags")):
        assert torch.equal(a, b), f"mode {mode} bs {bs}: {name} differ from dstill_verify"
    return ref


@pytest.mark.parametrize("mode,big,small", [
    (bd.VERIFY_RS, (32, 15, 151936), (5, 15, 151936)),
    (bd.VERIFY_GREEDY, (16, 15, 151936), (1, 15, 151936)),
    (bd.VERIFY_RS, (9, 7, 5003), (2, 3, 1024)),
])
def test_noalloc_matches_workspace_call(mode, big, small):
    for i, (bs, gamma, V) in enumerate((big, small)):
        zt, zd, y, lse = _inputs(mode, bs, gamma, V, seed=20 + i)
        _, tau, _ = _both(mode, zt, zd, y, lse, seed=3, cycle=i)
        assert (tau.cpu() >= 1).all() and (tau.cpu() <= gamma + 1).all()


def test_noalloc_refuses_shape_beyond_scratch():
    dev = device()
    need = bd.verify_workspace_bytes(7000, 15, 151936)
    assert need > bd.NOALLOC_SCRATCH_BYTES
    # the shape check happens before the device is touched: tiny dummy tensors
    t = torch.zeros(1, dtype=torch.int32, device=dev)
    zt = torch.zeros((1, 1, 1), dtype=torch.float32, device=dev)
    lib = bd._lib.load()
    import ctypes
    p = ctypes.c_void_p(t.data_ptr())
    code = lib.dstill_verify_noalloc(bd.VERIFY_GREEDY, 7000, 15, 151936, 1.0, 0, 0, p, None,
                                     None, ctypes.c_void_p(zt.data_ptr()), bd.F32, p, p, p,
                                     None)
    assert code == bd._lib.EWORKSPACE
    assert b"scratch" in lib.dstill_last_error()
