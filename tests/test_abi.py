"""The C-ABI library builds, loads and exports every symbol include/dstill.h
declares; host-side argument checks reject bad calls before any launch.

No GPU is needed: every call here fails validation (or is a pure size query)
before the library touches the HIP runtime's device functions.
"""

import ctypes
import os
import re

import pytest

from block_diffusion_speculative_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.ensure_built()


def _declared():
    txt = open(os.path.join(ROOT, "include", "dstill.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dstill_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dstill_version() == 100


def _cfg(**kw):
    base = dict(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, mlp=1408,
                vocab=5003, n_feat_layers=3, target_hidden=384, max_block=16,
                mask_token_id=5002, qk_norm=1, dtype=_lib.BF16, rms_eps=1e-6, rope_theta=1e6)
    base.update(kw)
    return _lib.Config(**base)


def test_create_rejects_bad_configs(lib):
    h = ctypes.c_void_p()
    layers = (_lib.LayerWeights * 2)()
    w = _lib.Weights(embed=1, lm_head=1, w_fuse=1, g_fuse=1, g_final=1, layers=layers)
    assert lib.dstill_create(None, ctypes.byref(w), ctypes.byref(h)) == _lib.EINVAL
    for kw, code in [(dict(head_dim=96), _lib.EUNSUPPORTED), (dict(n_kv_heads=3), _lib.ESHAPE),
                     (dict(max_block=17), _lib.EUNSUPPORTED), (dict(dtype=7), _lib.EUNSUPPORTED),
                     (dict(mlp=1400), _lib.EUNSUPPORTED), (dict(mask_token_id=5003), _lib.ESHAPE),
                     (dict(vocab=1), _lib.ESHAPE)]:
        c = _cfg(**kw)
        assert lib.dstill_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == code, kw
        assert lib.dstill_last_error()
    # layer pointers null -> EINVAL
    c = _cfg()
    assert lib.dstill_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == _lib.EINVAL


def test_create_and_size_queries_without_launching(lib):
    c = _cfg()
    L = (_lib.LayerWeights * 2)()
    for i in range(2):
        for f, _t in _lib.LayerWeights._fields_:
            setattr(L[i], f, 4096)
    w = _lib.Weights(embed=4096, lm_head=4096, w_fuse=4096, g_fuse=4096, g_final=4096, layers=L)
    h = ctypes.c_void_p()
    assert lib.dstill_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == _lib.OK
    n = ctypes.c_size_t()
    assert lib.dstill_kv_bytes(ctypes.byref(c), 3, 128, ctypes.byref(n)) == _lib.OK
    assert n.value == 3 * 2 * 128 * 128 * 2
    assert lib.dstill_kv_bytes(ctypes.byref(c), 3, 104, ctypes.byref(n)) == _lib.ESHAPE
    lim = _lib.Limits(max_batch=3, max_copies=2, max_ctx=1029, max_inject_rows=77,
                      max_head_rows=45)
    assert lib.dstill_workspace_bytes(h, ctypes.byref(lim), ctypes.byref(n)) == _lib.OK
    assert n.value > 0
    # calls that fail validation enqueue nothing and need no device
    kvp = (ctypes.c_void_p * 2)(4096, 4096)
    kv = _lib.KV(k=kvp, v=kvp, max_batch=3, cap=128)
    s = _lib.Sample(mode=0, temperature=1.0, seed=0, cycle=0)
    assert lib.dstill_block_draft(h, 4096, 4096, 4, 16, 1, 50, ctypes.byref(kv), 4096, None,
                                  4096, 10**9, None) == _lib.ESHAPE      # bs > max_batch
    assert lib.dstill_block_draft(h, 4096, 4096, 2, 17, 1, 50, ctypes.byref(kv), 4096, None,
                                  4096, 10**9, None) == _lib.ESHAPE      # block > max_block
    assert lib.dstill_block_draft(h, 4096, 4096, 2, 16, 1, 50, ctypes.byref(kv), 4096, None,
                                  4096, 1, None) == _lib.EWORKSPACE
    assert lib.dstill_lm_head_argmax(h, 4096, 15, 15, 16, ctypes.byref(s), 4096, None, None,
                                     None, None, None, 4096, 8, None) == _lib.EWORKSPACE
    s.temperature = 0.0
    assert lib.dstill_lm_head_argmax(h, 4096, 15, 15, 16, ctypes.byref(s), 4096, None, None,
                                     None, None, None, 4096, 10**9, None) == _lib.EINVAL
    assert lib.dstill_inject_kv(h, 4096, 4096, 4096, -1, ctypes.byref(kv), 4096, 10**9,
                                None) == _lib.ESHAPE
    assert lib.dstill_inject_kv(h, 4096, 4096, 4096, 5, ctypes.byref(kv), 4096, 8,
                                None) == _lib.EWORKSPACE
    assert lib.dstill_destroy(h) == _lib.OK


def test_verify_checks(lib):
    n = ctypes.c_size_t()
    assert lib.dstill_verify_workspace_bytes(32, 15, 151936, ctypes.byref(n)) == _lib.OK
    assert n.value > 0
    assert lib.dstill_verify_workspace_bytes(32, 64, 151936, ctypes.byref(n)) == _lib.ESHAPE
    args = [15, 1000, 1.0, 0, 0, 4096, 4096, 4096, 4096, 0, 4096, 4096, 4096, 4096]
    assert lib.dstill_verify(3, 2, *args, 10**9, None) == _lib.EINVAL           # mode
    assert lib.dstill_verify(1, 2, 15, 1000, 1.0, 0, 0, 4096, None, None, 4096, 0, 4096, 4096,
                             4096, 4096, 10**9, None) == _lib.EINVAL            # RS without q
    assert lib.dstill_verify(0, 2, *args, 16, None) == _lib.EWORKSPACE
    assert lib.dstill_verify(0, 2, 15, 1000, 1.0, 0, 0, 4096, None, None, 4096, 5, 4096, 4096,
                             4096, 4096, 10**9, None) == _lib.EUNSUPPORTED      # dtype
    assert lib.dstill_verify(0, 0, *args, 0, None) == _lib.OK                   # empty batch
