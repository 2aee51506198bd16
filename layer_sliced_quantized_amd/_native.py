"""ctypes binding of libslq (include/slice.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libslq.so.  PyTorch provides device memory and streams.  If the
library is missing this module raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libslq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "slice.h")

SLICE_OK, SLICE_EINVAL, SLICE_ESHAPE, SLICE_ERANGE, SLICE_ESTATE, SLICE_EHIP, SLICE_ENOSYS = 0, -1, -2, -3, -4, -5, -6
Q4_0, Q8_0 = 2, 8

TENSOR_IDS = {
    "attn_norm": 0, "ffn_norm": 1,
    "dn_q": 10, "dn_k": 11, "dn_v": 12, "dn_a": 13, "dn_b": 14, "dn_z": 15, "dn_out": 16,
    "wq": 20, "wg": 21, "wk": 22, "wv": 23, "wo": 24, "q_norm": 25, "k_norm": 26,
    "w_gate": 30, "w_up": 31, "w_down": 32,
    "embed": 40, "head": 41, "out_norm": 42,
    "dn_conv": 17, "dn_alog": 18, "dn_dtb": 19, "dn_norm": 28,
    "mtp_fc": 43, "mtp_norm_e": 44, "mtp_norm_h": 45,
}


class SliceConfig(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
        ("layer_begin", ctypes.c_int32), ("layer_end", ctypes.c_int32),
        ("attn_period", ctypes.c_int32),
        ("dn_heads", ctypes.c_int32), ("dn_dk", ctypes.c_int32), ("dn_dv", ctypes.c_int32),
        ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("rope_dims", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("qk_norm", ctypes.c_int32), ("attn_gate", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("dn_a_scale", ctypes.c_float), ("dn_a_bias", ctypes.c_float),
        ("dn_b_scale", ctypes.c_float), ("dn_z_scale", ctypes.c_float),
        ("ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("has_embed", ctypes.c_int32), ("has_head", ctypes.c_int32),
        ("tied_head", ctypes.c_int32),
        ("max_seq", ctypes.c_int32), ("max_verify", ctypes.c_int32),
        ("qtype", ctypes.c_int32), ("io_fp32", ctypes.c_int32),
        ("dn_variant", ctypes.c_int32), ("dn_k_heads", ctypes.c_int32), ("dn_conv", ctypes.c_int32),
        ("has_mtp", ctypes.c_int32), ("max_prefill", ctypes.c_int32),
    ]


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("rope_dims", ctypes.c_int32), ("rope_theta", ctypes.c_double),
        ("qk_norm", ctypes.c_int32), ("has_gate", ctypes.c_int32), ("eps", ctypes.c_float),
        ("max_seq", ctypes.c_int32), ("q_norm_dev", ctypes.c_void_p), ("k_norm_dev", ctypes.c_void_p),
    ]


class SliceError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libslq error {code}: {msg}")
        self.code = code


_lib = None

_V = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "slq_packed_bytes": (_SZ, [_I, _I64, _I64]),
    "slq_repack": (_I, [_I, _V, _I64, _I64, _V, _V]),
    "slq_dequant": (_I, [_I, _V, _I64, _I64, _V, _V]),
    "slq_gemv_workspace_bytes": (_SZ, [_I, _I64, _I64, _I]),
    "slq_gemv": (_I, [_I, _V, _I64, _I64, _I, _V, _V, _V, _SZ, _V]),
    "slq_gemv_noalloc": (_I, [_I, _V, _I64, _I64, _I, _V, _V, _V]),
    "slq_read_probe": (_I, [_V, _SZ, _V, _V]),
    "slq_dn_step": (_I, [_I, _I, _I, _I, _V, _V, _V, _V]),
    "slq_dn_state_layout": (_I, [_I, _I, _I, _V, _V, _I, _V]),
    "slq_attn_workspace_bytes": (_SZ, [ctypes.POINTER(AttnDesc), _I]),
    "slq_attn_prepare": (_I, [ctypes.POINTER(AttnDesc), _V, _SZ, _V]),
    "slq_attn_decode": (_I, [ctypes.POINTER(AttnDesc), _I, _I, _V, _V, _V, _V, _V, _SZ, _V]),
    "slq_kv_layout": (_I, [_I, _I, _I, _I, _V, _V, _V, _V, _I, _V]),
    "slice_weights_bytes": (_SZ, [ctypes.POINTER(SliceConfig)]),
    "slice_workspace_bytes": (_SZ, [ctypes.POINTER(SliceConfig)]),
    "slice_load": (_I, [ctypes.POINTER(SliceConfig), _V, _V, _V, ctypes.POINTER(_V)]),
    "slice_set_tensor": (_I, [_V, _I, _I, _V, _SZ, _V]),
    "slice_tensor_info": (_I, [ctypes.POINTER(SliceConfig), _I, _I, ctypes.POINTER(ctypes.c_int64),
                               ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32),
                               ctypes.POINTER(ctypes.c_size_t)]),
    "slq_debug_override": (_I, [ctypes.c_char_p, _I]),
    "slice_reset": (_I, [_V, _I, _V]),
    "slice_decode": (_I, [_V, _V, _V, _V]),
    "slice_decode_profiled": (_I, [_V, _V, _V, ctypes.POINTER(_I), ctypes.POINTER(ctypes.c_float), _I, _V]),
    "slice_run_gemv_op": (_I, [_V, _I, _V]),
    "slice_verify": (_I, [_V, _I, _V, _V, _V]),
    "slice_commit": (_I, [_V, _I, _V]),
    "slice_prefill": (_I, [_V, _I, _V, _V, _V]),
    "slice_embed": (_I, [_V, _V, _V, _V]),
    "slice_head_argmax": (_I, [_V, _V, _V, _V, _V]),
    "slice_mtp_input": (_I, [_V, _V, _V, _V, _V]),
    "slice_position": (_I, [_V]),
    "slice_sync_check": (_I, [_V, _V]),
    "slice_free": (None, [_V]),
    "slice_last_error": (ctypes.c_char_p, []),
    "slice_dbg_set_state": (_I, [_V, _I, _V, _V]),
    "slice_dbg_get_state": (_I, [_V, _I, _V, _V]),
    "slice_dbg_get_conv": (_I, [_V, _I, _V, _V]),
    "slice_dbg_set_conv": (_I, [_V, _I, _V, _V]),
    "slice_dbg_set_kv": (_I, [_V, _I, _V, _V, _I, _V]),
    "slice_dbg_get_kv": (_I, [_V, _I, _V, _V, _I, _V]),
    "slice_dbg_get_hidden": (_I, [_V, _V, _I, _V]),
}


def lib() -> ctypes.CDLL:
    """The loaded libslq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m layer_sliced_quantized_amd.build` "
                              "(hipcc, gfx950) first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(rc: int) -> None:
    if rc != SLICE_OK:
        msg = lib().slice_last_error()
        raise SliceError(rc, msg.decode() if msg else "")


def exported_names() -> list:
    return list(_SIGS)
