"""ctypes view of the C ABI in include/dstill.h.

Only argument marshalling lives here: every step of the path runs in the HIP
kernels of libdstill.so.  Loading fails loudly when the library is missing;
there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_uint32, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdstill.so")

# status codes and constants (mirror include/dstill.h)
OK, EINVAL, ESHAPE, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
HEAD_ARGMAX, HEAD_GUMBEL, HEAD_SHARED_GUMBEL = 0, 1, 2
VERIFY_GREEDY, VERIFY_RS = 0, 1
FLAG_NEAR_TIE_TARGET = 1
FLAG_NEAR_THRESHOLD = 2
FLAG_NEAR_TIE_SAMPLE = 4
FLAG_ZERO_RESIDUAL = 8
FLAG_BAD_INPUT = 16
FLAG_CTX_CLAMPED = 32
NEAR = 1e-5
NOALLOC_SCRATCH_BYTES = 4 << 20

# every symbol the header declares
EXPORTS = [
    "dstill_create", "dstill_destroy", "dstill_kv_bytes", "dstill_workspace_bytes",
    "dstill_inject_kv", "dstill_block_draft", "dstill_lm_head_argmax",
    "dstill_verify_workspace_bytes", "dstill_verify", "dstill_verify_noalloc",
    "dstill_dloop_branches",
    "dstill_dloop_merge", "dstill_verify_branches_workspace_bytes", "dstill_verify_branches",
    "dstill_spot_verify", "dstill_refine_commit", "dstill_last_error", "dstill_version",
]


class Config(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "mlp", "vocab",
        "n_feat_layers", "target_hidden", "max_block", "mask_token_id", "qk_norm", "dtype")] + [
        ("rms_eps", c_float), ("rope_theta", c_float), ("swa_window", c_int32),
        ("full_attn_mask", c_uint32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "attn_norm", "wqkv", "q_norm", "k_norm", "wo", "mlp_norm", "w_gate_up", "w_down")]


class Weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("w_fuse", c_void_p),
                ("g_fuse", c_void_p), ("g_final", c_void_p),
                ("layers", POINTER(LayerWeights))]


class KV(ctypes.Structure):
    _fields_ = [("k", POINTER(c_void_p)), ("v", POINTER(c_void_p)),
                ("max_batch", c_int32), ("cap", c_int32)]


class Limits(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "max_batch", "max_copies", "max_ctx", "max_inject_rows", "max_head_rows")]


class Sample(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("temperature", c_float), ("seed", c_uint64),
                ("cycle", c_uint64)]


_lib = None


class DstillError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def _declare(lib):
    vp, i32, sz = c_void_p, c_int32, c_size_t
    sig = {
        "dstill_create": ([POINTER(Config), POINTER(Weights), POINTER(c_void_p)], c_int32),
        "dstill_destroy": ([vp], c_int32),
        "dstill_kv_bytes": ([POINTER(Config), i32, i32, POINTER(c_size_t)], c_int32),
        "dstill_workspace_bytes": ([vp, POINTER(Limits), POINTER(c_size_t)], c_int32),
        "dstill_inject_kv": ([vp, vp, vp, vp, i32, POINTER(KV), vp, sz, vp], c_int32),
        "dstill_block_draft": ([vp, vp, vp, i32, i32, i32, i32, POINTER(KV), vp, vp, vp, sz, vp],
                               c_int32),
        "dstill_lm_head_argmax": ([vp, vp, i32, i32, i32, POINTER(Sample), vp, vp, vp, vp, vp, vp,
                                   vp, sz, vp], c_int32),
        "dstill_verify_workspace_bytes": ([i32, i32, i32, POINTER(c_size_t)], c_int32),
        "dstill_verify": ([i32, i32, i32, i32, c_float, c_uint64, c_uint64, vp, vp, vp, vp, i32,
                           vp, vp, vp, vp, sz, vp], c_int32),
        "dstill_verify_noalloc": ([i32, i32, i32, i32, c_float, c_uint64, c_uint64, vp, vp, vp, vp,
                                   i32, vp, vp, vp, vp], c_int32),
        "dstill_dloop_branches": ([i32, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp], c_int32),
        "dstill_dloop_merge": ([i32, i32, i32, vp, vp, vp, vp, vp], c_int32),
        "dstill_verify_branches_workspace_bytes": ([i32, i32, i32, i32, POINTER(c_size_t)],
                                                   c_int32),
        "dstill_verify_branches": ([i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp],
                                   c_int32),
        "dstill_spot_verify": ([i32, i32, i32, i32, c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, vp, vp], c_int32),
        "dstill_refine_commit": ([i32, i32, i32, i32, vp, vp, vp, vp, vp, vp], c_int32),
        "dstill_last_error": ([], ctypes.c_char_p),
        "dstill_version": ([], c_int32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res


def load(path: str = LIB_PATH):
    """Load libdstill.so (once).  Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m block_diffusion_speculative_kv_amd.build`"
            " (the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    _declare(lib)
    _lib = lib
    return lib


def ensure_built():
    """Build the library if it does not exist yet, then load it."""
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    return load()


def check(code: int, fn: str):
    if code != OK:
        msg = load().dstill_last_error()
        raise DstillError(code, fn, msg.decode() if msg else "")
