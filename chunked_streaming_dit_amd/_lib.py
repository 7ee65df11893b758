"""ctypes binding of libditchunk (include/ditchunk.h, include/ditchunk_ops.h).

Argument marshalling only: every computation runs in the HIP kernels of the library.
PyTorch supplies device memory (tensors) and the HIP stream.  If the library is not
built, importing the binding raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libditchunk.so")

DIT_OK, DIT_EINVAL, DIT_ESHAPE, DIT_ESTATE, DIT_EWORKSPACE, DIT_EHIP = 0, -1, -2, -3, -4, -5
DIT_F32, DIT_BF16 = 0, 1
DITK_ACT_NONE, DITK_ACT_GELU, DITK_OUT_F32 = 0, 1, 2
DIT_TIME_ATTN, DIT_TIME_GEMM, DIT_TIME_ELEM = 0, 1, 2

# Weight table order of ditchunk.h (DIT_W_* then DIT_WB_* per block).
GLOBAL_ORDER = ("pe.w", "pe.b", "t1.w", "t1.b", "t2.w", "t2.b", "fmod.w", "fmod.b", "fin.w", "fin.b")
BLOCK_ORDER = ("mod.w", "mod.b", "qkv.w", "qkv.b", "gq", "gk", "o.w", "o.b", "cq.w", "cq.b",
               "ck.w", "ck.b", "cv.w", "cv.b", "gcq", "gck", "co.w", "co.b", "fc1.w", "fc1.b",
               "fc2.w", "fc2.b")


class DitConfig(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int), ("D", ctypes.c_int), ("H", ctypes.c_int), ("dh", ctypes.c_int),
                ("mlp_ratio", ctypes.c_int), ("c_p", ctypes.c_int), ("c_c", ctypes.c_int),
                ("cond_up", ctypes.c_int), ("d_a", ctypes.c_int), ("dtype", ctypes.c_int),
                ("max_tokens", ctypes.c_int), ("max_ref", ctypes.c_int), ("max_bnd", ctypes.c_int),
                ("max_audio", ctypes.c_int), ("eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


class DitGrid(ctypes.Structure):
    _fields_ = [("t0", ctypes.c_int), ("frames", ctypes.c_int), ("h", ctypes.c_int), ("w", ctypes.c_int)]


class DitError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libditchunk error {code}: {msg}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None

DIT_AUDIO_HELD = -1
DIT_MOD_TABLE_MAX = 16
DITK_PROBE_SINK_FLOATS = 512 * 256
P = ctypes.c_void_p
I = ctypes.c_int
Dbl = ctypes.c_double

_SIGS = {
    "dit_weight_count": (I, [ctypes.POINTER(DitConfig)]),
    "dit_state_bytes": (ctypes.c_size_t, [ctypes.POINTER(DitConfig)]),
    "dit_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(DitConfig)]),
    "dit_create": (I, [ctypes.POINTER(DitConfig), ctypes.POINTER(P), P, ctypes.c_size_t, P,
                       ctypes.c_size_t, P, ctypes.POINTER(P)]),
    "dit_destroy": (I, [P]),
    "audio_kv_precompute": (I, [P, P, I]),
    "dit_modulation_table": (I, [P, ctypes.POINTER(Dbl), I]),
    "dit_block_weight_bytes": (ctypes.c_size_t, [ctypes.POINTER(DitConfig)]),
    "dit_weight_stream": (I, [P, ctypes.POINTER(P), P, ctypes.c_size_t, I]),
    "ref_kv_precompute": (I, [P, P, DitGrid]),
    "boundary_kv_carry": (I, [P, P, DitGrid]),
    "interp_anchor_kv": (I, [P, P, DitGrid, I]),
    "dit_chunk_step": (I, [P, P, P, P, I, DitGrid, Dbl, Dbl, P]),
    "dit_chunk_step_carry": (I, [P, P, P, P, I, DitGrid, Dbl, Dbl, P]),
    "fm_euler_step": (I, [P, P, Dbl, ctypes.c_longlong, P]),
    "fm_noise_to": (I, [P, P, P, Dbl, ctypes.c_longlong, P]),
    "dit_last_error": (ctypes.c_char_p, []),
    "dit_timing_enable": (I, [P, I]),
    "dit_timing_read": (I, [P, I, ctypes.POINTER(I), ctypes.POINTER(Dbl), ctypes.POINTER(Dbl)]),
    "ditk_linear": (I, [I, P, P, P, I, I, I, I, P, P]),
    "ditk_linear_residual": (I, [I, P, P, P, P, I, I, I, P, P, ctypes.c_longlong, P]),
    "ditk_rmsnorm_modulate": (I, [I, P, I, I, P, P, Dbl, P, P]),
    "ditk_qknorm_rope": (I, [I, I, I, I, P, P, P, I, P, P, I, DitGrid, Dbl, Dbl, Dbl, P, P, P, I, P]),
    "ditk_attention": (I, [I, I, I, P, I, I, ctypes.POINTER(P), ctypes.POINTER(P),
                           ctypes.POINTER(I), ctypes.POINTER(I), I, P, I, I, P, P, Dbl, P, P]),
    "ditk_attention_noalloc": (I, [I, I, I, P, I, I, ctypes.POINTER(P), ctypes.POINTER(P),
                                   ctypes.POINTER(I), ctypes.POINTER(I), I, I, I, P, P, Dbl, P, P]),
    "ditk_attention_probs": (I, [I, P, I, P, I, I, I, P, P]),
    "ditk_modulation": (I, [I, I, I, Dbl, ctypes.POINTER(P), P, P, P, P]),
    "ditk_patch_input": (I, [I, P, I, I, P, I, I, DitGrid, P, P]),
    "ditk_patch_embed": (I, [P, I, I, P, I, I, DitGrid, P, P, P, I, P]),
    "ditk_probe_mfma": (I, [P, I, P, ctypes.c_longlong, ctypes.POINTER(Dbl), P]),
    "ditk_probe_copy": (I, [P, P, ctypes.c_longlong, P]),
}
EXPORTS = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """Load libditchunk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with chunked_streaming_dit_amd.build "
                              "(the HIP library is required; there is no fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def last_error() -> str:
    return lib().dit_last_error().decode()


def check(rc: int) -> None:
    if rc != DIT_OK:
        raise DitError(rc, last_error())
