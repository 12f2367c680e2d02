"""ctypes loader of libbd.so (the gfx950 HIP library built by build.py).

Loading fails loudly when the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbd.so")

BD_OK, BD_EINVAL, BD_EUNSUPPORTED, BD_ECAPACITY, BD_EHIP, BD_ESCRATCH = 0, 1, 2, 3, 4, 5
BD_F32, BD_BF16 = 0, 1

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class BdRows(ctypes.Structure):
    """Row map: logical row r -> buffer row (r // group) * stride + offset + r % group."""
    _fields_ = [("group", ctypes.c_int32), ("stride", ctypes.c_int32), ("offset", ctypes.c_int32)]


class BdGuard(ctypes.Structure):
    """Device-side condition of a call: it does nothing when no bits[b], b < n,
    has a bit of mask set."""
    _fields_ = [("bits", ctypes.c_void_p), ("mask", ctypes.c_uint64), ("n", ctypes.c_int32)]


class BdNextRows(ctypes.Structure):
    """The next step's input rows written by bd_lmhead_unmask_next."""
    _fields_ = [("embedding", ctypes.c_void_p), ("plant", ctypes.c_void_p), ("x", ctypes.c_void_p)]


# name -> (restype, argtypes)
SIGNATURES = {
    "bd_version": (ctypes.c_char_p, []),
    "bd_status_string": (ctypes.c_char_p, [c_int]),
    "bd_last_hip_error": (c_int, []),
    "bd_block_attn_workspace_size": (c_size_t, [c_int] * 8),
    "bd_block_attn": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int,
                              c_void_p, c_int, c_int,
                              c_void_p, c_void_p, c_void_p, c_int,
                              c_void_p, c_void_p, c_int,
                              c_float, c_void_p, c_void_p,
                              c_void_p, c_size_t, c_void_p]),
    "bd_block_attn_guarded": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_void_p, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p, c_int,
                                      c_void_p, c_void_p, c_int,
                                      c_float, c_void_p, c_void_p,
                                      c_void_p, c_size_t, ctypes.POINTER(BdGuard), c_void_p]),
    "bd_block_attn_noalloc": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_void_p, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p, c_int,
                                      c_void_p, c_void_p, c_int,
                                      c_float, c_void_p, c_void_p, c_void_p]),
    "bd_block_attn_noalloc_scratch_bytes": (c_size_t, []),
    "bd_lmhead_workspace_size": (c_size_t, [c_int] * 4),
    "bd_lmhead_confidence": (c_int, [c_int, c_int, c_int, c_int,
                                     c_void_p, c_int, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
    "bd_lmhead_confidence_rows": (c_int, [c_int, c_int, c_int, c_int,
                                          c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_int, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_size_t, c_void_p]),
    "bd_lmhead_unmask": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                 c_void_p, c_int, c_void_p, c_void_p, c_float, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_size_t, c_void_p]),
    "bd_lmhead_unmask_next": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_void_p, c_int, c_void_p, c_void_p, c_float, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      ctypes.POINTER(BdNextRows), c_void_p, c_size_t, c_void_p]),
    "bd_candidate_rows": (c_int, [c_int, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bd_threshold_unmask": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_float,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bd_threshold_unmask_tau": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bd_threshold_unmask_windows": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_float,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bd_copy_rows": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bd_probe_weight_stream": (c_int, [c_void_p, c_int, c_int, c_void_p, c_int, c_int, c_void_p]),
    "bd_persequence_schedule": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bd_kv_append": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "bd_embed_rows": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "bd_linear_workspace_size": (c_size_t, [c_int] * 4),
    "bd_linear": (c_int, [c_int, c_int, c_int, c_int, c_void_p, BdRows, c_void_p,
                          c_void_p, BdRows, c_void_p, BdRows, c_void_p, c_size_t, c_void_p]),
    "bd_linear_guarded": (c_int, [c_int, c_int, c_int, c_int, c_void_p, BdRows, c_void_p,
                                  c_void_p, BdRows, c_void_p, BdRows, c_void_p, c_size_t, ctypes.POINTER(BdGuard),
                                  c_void_p]),
    "bd_linear_residual_rmsnorm": (c_int, [c_int, c_int, c_int, c_int, c_void_p, BdRows, c_void_p, c_void_p,
                                           BdRows, c_float, c_void_p, BdRows, c_void_p, c_size_t, c_void_p]),
    "bd_qkv_proj_workspace_size": (c_size_t, [c_int] * 5),
    "bd_qkv_proj": (c_int, [c_int, c_int, c_int, c_void_p, BdRows,
                            c_void_p, c_int, c_void_p, BdRows,
                            c_void_p, c_void_p, c_int, c_void_p, BdRows, c_void_p, BdRows,
                            c_void_p, c_size_t, c_void_p]),
    "bd_qkv_proj_guarded": (c_int, [c_int, c_int, c_int, c_void_p, BdRows,
                                    c_void_p, c_int, c_void_p, BdRows,
                                    c_void_p, c_void_p, c_int, c_void_p, BdRows, c_void_p, BdRows,
                                    c_void_p, c_size_t, ctypes.POINTER(BdGuard), c_void_p]),
    "bd_qkv_proj_rope_workspace_size": (c_size_t, [c_int] * 5),
    "bd_qkv_proj_rope": (c_int, [c_int, c_int, c_int, c_void_p, BdRows,
                                 c_void_p, c_int, c_void_p, BdRows,
                                 c_void_p, c_void_p, c_int, c_void_p, BdRows, c_void_p, BdRows,
                                 c_int, c_void_p, c_int, c_int, c_float,
                                 c_void_p, c_size_t, c_void_p]),
    "bd_gate_up_swiglu": (c_int, [c_int, c_int, c_int, c_void_p, BdRows, c_void_p, c_int, c_void_p, BdRows,
                                  c_void_p]),
    "bd_gate_up_swiglu_rmsnorm": (c_int, [c_int, c_int, c_int, c_void_p, BdRows, c_float, c_void_p, c_int, c_void_p,
                                          BdRows, c_void_p]),
    "bd_train_attn_workspace_size": (c_size_t, [c_int] * 7),
    "bd_train_attn": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                              c_float, c_void_p, c_void_p, c_size_t, c_void_p]),
    "bd_masked_nll": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p]),
    "bd_rmsnorm": (c_int, [c_int, c_int, c_int, c_void_p, BdRows, c_float, c_void_p, BdRows, c_void_p]),
    "bd_rope": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, BdRows, c_void_p, c_int, c_float, c_void_p]),
    "bd_swiglu": (c_int, [c_int, c_int, c_int, c_void_p, BdRows, c_void_p, BdRows, c_void_p]),
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libbd.so not found at {LIB_PATH}; build it with "
                          "`python -m block_diffusion_decoding_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
