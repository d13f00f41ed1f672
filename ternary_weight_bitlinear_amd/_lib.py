"""ctypes loader for libbitnet_hip.so (the C ABI in include/bitnet.h).

The library must have been built ahead of time (``python -m
ternary_weight_bitlinear_amd.build``).  If it is missing, every entry point
raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import os

# BITNET_LIBRARY may name another build of the same library (the tests use it
# for the sanitized host build); by default the in-tree build is loaded.
LIBRARY = Path(os.environ.get("BITNET_LIBRARY") or Path(__file__).resolve().parent / "libbitnet_hip.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_NONFINITE = range(5)
F32, BF16, F16 = 0, 1, 2
MEM_HOST, MEM_DEVICE = 0, 1
I2S_STRIDED, I2S_CONSECUTIVE = 0, 1

# name -> (restype, argtypes), in the order of include/bitnet.h
_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
SIGNATURES = {
    "bitnet_abi_version": (_i32, []),
    "bitnet_padded_k": (_i64, [_i64]),
    "bitnet_packed_bytes": (_i64, [_i64, _i64]),
    "bitnet_pack_weights": (ctypes.c_int, [ctypes.c_int, _vp, _vp, ctypes.c_int, _i64, _i64, _i64,
                                           _vp, _i32, _vp, _vp, _vp, _vp]),
    "bitnet_pack_weights_static": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                                                  _vp, _vp]),
    "bitnet_act_quant": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp]),
    "bitnet_rmsnorm_act_quant": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp,
                                                ctypes.c_int, ctypes.c_float, _vp, _vp, _vp]),
    "bitnet_linear_forward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64,
                                             _vp, ctypes.c_int, _i64, _vp]),
    "bitnet_bitlinear_forward": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp,
                                                _i64, _vp, ctypes.c_int, _i64, _vp, _vp, _vp]),
    "bitnet_rmsnorm_bitlinear_forward": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp,
                                                        ctypes.c_int, ctypes.c_float, _vp, _vp, _i64, _vp,
                                                        ctypes.c_int, _i64, _vp, _vp, _vp]),
    "bitnet_group_table_bytes": (_i64, [_i32]),
    "bitnet_group_plan": (ctypes.c_int, [_vp, _vp, _i32, _i64, ctypes.c_int, ctypes.c_int, _vp, _i64, _vp]),
    "bitnet_group_plan_rmsnorm": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, ctypes.c_int, ctypes.c_int, _vp, _i64,
                                                 _vp]),
    "bitnet_group_plan_a16": (ctypes.c_int, [_vp, _vp, _i32, _i64, ctypes.c_int, _vp, _i64, _vp]),
    "bitnet_group_plan_a16_fp16": (ctypes.c_int, [_vp, _vp, _i32, _i64, ctypes.c_int, _vp, _i64, _vp]),
    "bitnet_group_plan_blocked": (ctypes.c_int, [_vp, _vp, _i32, _i64, ctypes.c_int, ctypes.c_int, _vp, _i64,
                                                 _vp]),
    "bitnet_bitlinear_grouped": (ctypes.c_int, [_vp, _vp]),
    "bitnet_group_plan_kernel": (ctypes.c_char_p, [_vp]),
    "bitnet_linear_a16": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _i64, _vp,
                                         ctypes.c_int, _i64]),
    "bitnet_i2s_bytes": (_i64, [_i64, _i64]),
    "bitnet_i2s_import": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _i64, _i64, ctypes.c_int, _vp, _vp]),
    "bitnet_i2s_export": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp]),
    "bitnet_save_packed": (ctypes.c_int, [ctypes.c_char_p, _vp, _vp, _i64, _i64, _vp, _vp, _i32]),
    "bitnet_load_packed": (ctypes.c_int, [ctypes.c_char_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "bitnet_block_count": (_i64, [_i64]),
    "bitnet_pack_weights_blocked": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _vp]),
    "bitnet_linear_blocked_forward": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp,
                                                     ctypes.c_int, _i64]),
    "bitnet_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bitnet_last_error": (ctypes.c_char_p, []),
}


class GroupItem(ctypes.Structure):
    """bitnet_group_item_t."""
    _fields_ = [("x", _vp), ("ldx", _i64), ("packed", _vp), ("w_scale", _vp), ("y", _vp),
                ("ldy", _i64), ("N", _i64), ("K", _i64)]


class GroupNorm(ctypes.Structure):
    """bitnet_group_norm_t."""
    _fields_ = [("up", _vp), ("norm_w", _vp), ("norm_dtype", ctypes.c_int), ("eps", ctypes.c_float)]


class GroupPlan(ctypes.Structure):
    """bitnet_group_plan_t (opaque)."""
    _fields_ = [("opaque", _i64 * 8)]


class BitnetError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIBRARY.exists():
            raise RuntimeError(f"{LIBRARY} is not built; run `python -m ternary_weight_bitlinear_amd.build`")
        handle = ctypes.CDLL(str(LIBRARY))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != OK:
        detail = lib().bitnet_last_error().decode() or lib().bitnet_status_string(status).decode()
        raise BitnetError(status, detail)
