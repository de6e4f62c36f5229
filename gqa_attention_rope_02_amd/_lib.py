"""ctypes loader for the in-tree ``libllama_attn.so`` (see include/llama_attn.h).

The library is built by ``python -m gqa_attention_rope_02_amd.build``. There is
no fallback: if the shared library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllama_attn.so")

_c_i64_p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_i = ctypes.c_int

# name -> (argtypes, restype), mirroring include/llama_attn.h
SIGNATURES = {
    "la_status_str": ([_i], ctypes.c_char_p),
    "la_version": ([], _i),
    "rope_qk": ([_vp, _vp, _c_i64_p, _c_i64_p, _vp, _vp, _c_i64_p, _c_i64_p, _i,
                 _i, _i, _i, _i, _i, _vp, ctypes.c_double, _i, _vp], _i),
    "rope_qk_backward": ([_vp, _vp, _c_i64_p, _c_i64_p, _vp, _vp, _c_i64_p, _c_i64_p, _i,
                          _i, _i, _i, _i, _i, _vp, ctypes.c_double, _i, _vp], _i),
    "gqa_attention_backward": ([_vp] * 10 + [_i, _i, _i, _i, _i, _i] + [_c_i64_p] * 8
                               + [_vp, _i, ctypes.c_float, _vp, _vp], _i),
    "gqa_prefill": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                     _c_i64_p, _c_i64_p, _c_i64_p, _c_i64_p, _vp, _i, ctypes.c_float, _vp], _i),
    "gqa_prefill_rope": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                          _c_i64_p, _c_i64_p, _c_i64_p, _c_i64_p, _vp, _i, ctypes.c_float,
                          _vp, ctypes.c_double, _i, _vp], _i),
    "gqa_prefill_chunk": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                           _c_i64_p, _c_i64_p, _c_i64_p, _c_i64_p, _vp, _i, ctypes.c_float,
                           _vp, ctypes.c_double, _i, _vp], _i),
    "gqa_prefill_split": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                           _c_i64_p, _c_i64_p, _c_i64_p, _c_i64_p, _vp, _i, ctypes.c_float,
                           _vp, ctypes.c_double, _i, _i, _i, _vp, _vp, _vp], _i),
    "gqa_prefill_ring_step": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                               _c_i64_p, _c_i64_p, _c_i64_p, _vp, _i, ctypes.c_float, _vp,
                               ctypes.c_double, _i, _i, _vp], _i),
    "gqa_prefill_ring_step_final": ([_vp, _vp, _vp, _vp, _vp, _vp, _c_i64_p, _vp, _i, _i, _i, _i, _i,
                                     _i, _i, _i, _i, _c_i64_p, _c_i64_p, _c_i64_p, _vp, _i,
                                     ctypes.c_float, _vp, ctypes.c_double, _i, _i, _vp], _i),
    "gqa_prefill_ring_finalize": ([_vp, _vp, _vp, _c_i64_p, _vp, _i, _i, _i, _i, _i, _vp], _i),
    "gqa_decode": ([_vp, _c_i64_p, _vp, _vp, _c_i64_p, _vp, _i, _i, _i, _i, _i, _i, _i,
                    ctypes.c_float, _vp, _vp, _vp], _i),
    "gqa_decode_paged": ([_vp, _c_i64_p, _vp, _vp, _c_i64_p, _i, _vp, _i, _vp, _i, _i, _i, _i,
                          _i, _i, _i, ctypes.c_float, _vp, _vp, _vp], _i),
    "gqa_decode_combine": ([_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _c_i64_p, _vp, _i, _vp], _i),
    "gqa_decode_noalloc": ([_vp, _c_i64_p, _vp, _vp, _c_i64_p, _vp, _i, _i, _i, _i, _i, _i,
                            ctypes.c_float, _vp, _c_i64_p, _vp, _i, _vp], _i),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load (once) and return the C-ABI library with its signatures set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m gqa_attention_rope_02_amd.build` "
            "(the attention path has no non-HIP implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (argtypes, restype) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _lib = lib
    return lib


def i64_array(values):
    """A ctypes int64 array (for the stride arguments)."""
    arr = (ctypes.c_int64 * len(values))(*[int(v) for v in values])
    return arr
