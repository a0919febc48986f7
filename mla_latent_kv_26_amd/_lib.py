"""ctypes loader for libmla_latent_kv.so (the C ABI in include/mla.h).

Raises at import time if the library has not been built: there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MLA_LIB_PATH", os.path.join(_HERE, "libmla_latent_kv.so"))

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE = 3
MLA_ERR_HIP = 4
DTYPE_F32 = 0
DTYPE_BF16 = 1
CACHE_SAME = 0
CACHE_FP8_E4M3 = 1


class MLAConfigC(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("qk_nope_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("q_lora_rank", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("rms_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("kv_groups", ctypes.c_int32),
        ("split_workgroups", ctypes.c_int32),
        ("prefill_attention", ctypes.c_int32),
        ("decode_attention", ctypes.c_int32),
    ]


class MLAError(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        self.status = status
        self.func = func
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {message}")


STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
                3: "MLA_ERR_WORKSPACE", 4: "MLA_ERR_HIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} not found: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()' or "
        "python mla_latent_kv_26_amd/build.py)")

# The library must bind to the same HIP runtime instance as torch (streams
# and device pointers cross this boundary), so torch's runtime is loaded
# first; the library's libamdhip64.so.7 dependency then resolves to it.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int32
_CFG = ctypes.POINTER(MLAConfigC)
_IP = ctypes.c_void_p          # int32 device pointers are passed as raw addresses
_FP = ctypes.c_void_p
_SZ = ctypes.c_size_t

SIGNATURES = {
    "mla_abi_version": (_I, []),
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_validate_config": (_I, [_CFG]),
    "mla_cache_row_elems": (ctypes.c_int64, [_CFG]),
    "mla_cache_bytes_per_token": (ctypes.c_int64, [_CFG]),
    "mla_rope_table": (_I, [_CFG, _I, ctypes.POINTER(ctypes.c_float)]),
    "mla_decode_workspace_size": (_I, [_CFG, _I, _I, ctypes.POINTER(_SZ)]),
    "mla_decode": (_I, [_CFG, _P, _P, _P, _P, _P, _I, _IP, _I, _IP, _I, _I, _P, _P, _SZ, _P]),
    "mla_decode_noalloc": (_I, [_CFG, _P, _P, _P, _P, _P, _I, _IP, _I, _IP, _I, _I, _P, _P]),
    "mla_absorb_query": (_I, [_CFG, _P, _P, _P, _I, _P, _P]),
    "mla_latent_attention": (_I, [_CFG, _P, _P, _I, _IP, _I, _IP, _I, _I, _P, _P, _SZ, _P]),
    "mla_attention_partials": (_I, [_CFG, _P, _P, _I, _IP, _I, _IP, _I, _I, _P, _SZ, _P]),
    "mla_combine_output": (_I, [_CFG, _P, _I, _I, _P, _P, _SZ, _P]),
    "mla_output_projection": (_I, [_CFG, _P, _P, _I, _P, _P]),
    "mla_cache_append_workspace_size": (_I, [_CFG, _I, ctypes.POINTER(_SZ)]),
    "mla_cache_append": (_I, [_CFG, _P, _P, _FP, _FP, _I, _IP, _IP, _I, _P, _I, _P, _SZ, _P]),
    "mla_prefill_workspace_size": (_I, [_CFG, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "mla_prefill_attention_form": (_I, [_CFG, _I, _I, ctypes.POINTER(_I)]),
    "mla_output_gate_workspace_size": (_I, [_CFG, _I, ctypes.POINTER(_SZ)]),
    "mla_output_gate_projection": (_I, [_CFG, _P, _P, _P, _P, _I, _P, _P, _SZ, _P]),
    "mla_prefill": (_I, [_CFG, _P, _P, _P, _FP, _P, _P, _FP, _P, _P, _FP, _I, _P, _I, _IP, _I,
                         _IP, _I, _I, _I, _P, _P, _SZ, _P]),
    "mla_probe_sink_bytes": (_SZ, []),
    "mla_probe_hbm_read": (_I, [_P, _SZ, _I, _P, _P]),
    "mla_probe_mfma": (_I, [_I, _I, _P, _P]),
    "mla_probe_lds_read": (_I, [_I, _I, _P, _P]),
}

for _name, (_res, _args) in SIGNATURES.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def last_error() -> str:
    return lib.mla_last_error().decode()


def check(status: int, func: str) -> None:
    if status != MLA_OK:
        raise MLAError(status, func, last_error())
