"""ctypes view of the C-ABI declared in ``include/mla.h``.

Loads ``libmla_amd.so`` built in-tree by ``build.py``.  There is no fallback:
if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_amd.so")
PROBE_LIB_PATH = os.path.join(HERE, "libmla_probe.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, -1, -2, -3, -4
MLA_F32, MLA_BF16 = 0, 1
MLA_CACHE_DENSE, MLA_CACHE_INT4, MLA_CACHE_INT2 = 0, 1, 2


class MlaDims(ctypes.Structure):
    _fields_ = [
        ("n_heads", c_int32), ("d_model", c_int32), ("d_nope", c_int32), ("d_v", c_int32),
        ("d_c", c_int32), ("d_r", c_int32), ("rope_dims", c_int32), ("band", c_int32 * 3),
        ("rope_theta", c_float), ("softmax_scale", c_float), ("dtype", c_int32),
        ("cache_fmt", c_int32), ("qk_norm", c_int32), ("qk_norm_eps", c_float),
    ]


class MlaGeom(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32), ("grid_h", c_int32), ("grid_w", c_int32), ("window", c_int32),
        ("frames_per_block", c_int32),
    ]


_D = POINTER(MlaDims)
_G = POINTER(MlaGeom)
_I32P = POINTER(c_int32)

# name -> (restype, argtypes); one entry per function declared in include/mla.h
SIGNATURES = {
    "mla_cache_bytes": (c_size_t, [_D, _G]),
    "mla_cache_aux_bytes": (c_size_t, [_D, _G]),
    "mla_append_workspace_size": (c_size_t, [_D, _G, c_int32]),
    "mla_cache_append": (c_int, [_D, _G, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_size_t]),
    "mla_absorb_q": (c_int, [_D, _G, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_void_p]),
    "mla_fold_query_weights": (c_int, [_D, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "mla_absorb_q_folded": (c_int, [_D, _G, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p]),
    "mla_qk_norm_prepare": (c_int, [_D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_key_norm_workspace_size": (c_size_t, [_D, _G, c_int32]),
    "mla_cache_key_norm": (c_int, [_D, _G, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_size_t]),
    "mla_attention_workspace_size": (c_size_t, [_D, _G, c_int32]),
    "mla_attention": (c_int, [_D, _G, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t]),
    "mla_attention_noalloc": (c_int, [_D, _G, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_unabsorb_out": (c_int, [_D, _G, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p]),
    "mla_cache_dequant": (c_int, [_D, _G, c_void_p, c_void_p, c_void_p, c_void_p]),
    "mla_cache_rope_shift": (c_int, [_D, _G, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "mla_status_string": (c_char_p, [c_int]),
    "mla_last_error": (c_char_p, []),
    "mla_abi_version": (c_int, []),
}

# the measurement probes (include/mla_probe.h, libmla_probe.so)
PROBE_SIGNATURES = {
    "mla_probe_mfma": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "mla_probe_hbm_read": (c_int, [c_void_p, c_void_p, c_int64, c_int32, c_void_p]),
    "mla_probe_last_error": (c_char_p, []),
}

_lib = None
_probe_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m head_latent_attention_cache_amd.build` "
            "(the MLA path has no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def load_probe(path: str | None = None) -> ctypes.CDLL:
    """Load the measurement-probe library once; raise if it is not built."""
    global _probe_lib
    if _probe_lib is not None:
        return _probe_lib
    path = path or PROBE_LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m head_latent_attention_cache_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in PROBE_SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _probe_lib = lib
    return lib


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


def check(status: int) -> None:
    if status != MLA_OK:
        lib = load()
        raise MLAError(status, f"{lib.mla_status_string(status).decode()}: {lib.mla_last_error().decode()}")
