"""Shared helpers for the GPU parity tests: weight / input transfer to the
oracle and the comparison rules.

Comparison rules (the bar every GPU test applies):
* integer results (token ids, tau) are compared bit-exactly, except on rows
  or sequences where either side raised a near-tie flag (a top-2 score gap or
  |p/q - u| below 1e-5); those are counted and reported, never silently
  dropped;
* fp32 paths: |gpu - oracle| <= 1e-5 * max(1, |oracle|);
* bf16 paths: logits within 2e-2 absolute; intermediate bf16 tensors within a
  few bf16 units in the last place.
"""

from __future__ import annotations

import numpy as np
import torch

NEAR = 1e-5
NEAR_BITS = 1 | 2 | 4   # near-tie target, near threshold, near-tie sample


def to_np(t):
    """Host float64 (or int64) copy of a tensor, or of a nested dict/list."""
    if isinstance(t, dict):
        return {k: to_np(v) for k, v in t.items()}
    if isinstance(t, list):
        return [to_np(v) for v in t]
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16, torch.float32, torch.float64):
        return t.double().numpy()
    return t.long().numpy()


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def assert_close_rel(got, want, rel, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    err = np.abs(got - want) / np.maximum(1.0, np.abs(want))
    i = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.max() <= rel, (
        f"{what}: max scaled error {err.max():.3e} > {rel:g} at flat index {i} "
        f"(got {got.flat[i]!r}, want {want.flat[i]!r})")


def assert_close_abs(got, want, atol, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    err = np.abs(got - want)
    i = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.max() <= atol, (
        f"{what}: max abs error {err.max():.3e} > {atol:g} at flat index {i} "
        f"(got {got.flat[i]!r}, want {want.flat[i]!r})")


def assert_within_ulps(got, want, ulps, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    err = np.abs(got - want) / bf16_ulp(want)
    i = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.max() <= ulps, (
        f"{what}: {err.max():.2f} bf16 ulps > {ulps} at flat index {i} "
        f"(got {got.flat[i]!r}, want {want.flat[i]!r})")


def assert_bf16_rows_close(got, want, what):
    """bf16 tensors produced by rounding fp32 (kernel) and fp64 (oracle)
    values: the pre-rounding values differ by far less than the row scale, so
    each element may differ by one rounding of its own (2 ulps) plus a small
    fraction of the row's RMS (a rounding flip upstream, e.g. in a bf16 input
    of the projection, moves a value by ~1e-4 of the row scale)."""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    tol = 2 * bf16_ulp(want) + 2.0 ** -8 * rms
    err = np.abs(got - want) - tol
    i = int(np.argmax(err)) if err.size else 0
    assert err.size == 0 or err.max() <= 0, (
        f"{what}: error exceeds 2 ulps + rms/256 at flat index {i} "
        f"(got {got.flat[i]!r}, want {want.flat[i]!r})")


def compare_ids(gpu_ids, ref_ids, excluded, what):
    """Bit-exact id comparison outside the excluded (flagged) positions.
    Returns the number of excluded positions."""
    gpu_ids, ref_ids = np.asarray(gpu_ids), np.asarray(ref_ids)
    excluded = np.asarray(excluded, dtype=bool)
    bad = (gpu_ids != ref_ids) & ~excluded
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} mismatches outside the near-tie band, first at "
        f"{np.argwhere(bad)[0].tolist()}: gpu {gpu_ids[bad][0]} vs oracle {ref_ids[bad][0]}")
    return int(excluded.sum())


def device():
    import block_diffusion_speculative_kv_amd._lib as L
    L.load()
    return torch.device("cuda:0")
