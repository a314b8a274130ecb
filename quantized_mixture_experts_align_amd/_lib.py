"""ctypes binding of libmoe_w4a16.so (the C ABI declared in include/moe_w4a16.h).

Loading fails loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4a16.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ESIZE, MOE_EHIP = 0, -1, -2, -3, -4
QTYPE = {"int4_g128": 0, "nvfp4_g16": 1, "mxfp4_g32": 2, "int4zp_g128": 3, "int4zpf_g128": 4}
ACT = {"silu_mul": 0, "swiglu_alpha": 1, "relu2": 2}
GATED = {"silu_mul": True, "swiglu_alpha": True, "relu2": False}
PREP_GATE_UP, PREP_INTERLEAVED, PREP_PAD, PREP_ACT_ORDER = 0x1, 0x2, 0x4, 0x8
GEMM_AUTO, GEMM_DECODE, GEMM_MFMA = 0, 1, 2
NOALLOC_MAX_COUNTERS = 262144   # MOE_NOALLOC_MAX_COUNTERS


class MoeWeights(C.Structure):
    _fields_ = [
        ("qtype", C.c_int32), ("n_experts", C.c_int32), ("N", C.c_int32), ("K", C.c_int32),
        ("N_logical", C.c_int32), ("K_logical", C.c_int32), ("flags", C.c_uint32),
        ("reserved", C.c_int32), ("codes", C.c_void_p), ("scales", C.c_void_p),
        ("global_scale", C.c_void_p), ("bias", C.c_void_p), ("perm", C.c_void_p),
    ]


class MoeGemmConfig(C.Structure):
    _fields_ = [("kernel", C.c_int32), ("ng", C.c_int32), ("ksplit", C.c_int32),
                ("gemv_rows", C.c_int32), ("group_m", C.c_int32), ("block_order", C.c_void_p)]


class MoeRequantConfig(C.Structure):
    _fields_ = [("workgroups", C.c_int32), ("unroll", C.c_int32)]


class MoeError(RuntimeError):
    pass


_P, _I32, _I64, _SZ, _F = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
SIGNATURES = {
    "moe_last_error": (C.c_char_p, []),
    "moe_abi_version": (_I32, []),
    "moe_align_capacity": (C.c_int, [_I64, _I32, _I32, _I32, C.POINTER(_I64), C.POINTER(_I64)]),
    "moe_align": (C.c_int, [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "moe_align_sched": (C.c_int, [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "moe_w4a16_prepared_size": (C.c_int, [C.c_int, _I32, _I32, _I32, C.c_uint32, _I32,
                                          C.POINTER(_I32), C.POINTER(_I32), C.POINTER(_SZ)]),
    "moe_w4a16_prepare": (C.c_int, [C.c_int, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, C.c_uint32, _P,
                                    _SZ, C.POINTER(MoeWeights), _P]),
    "moe_permute_cols": (C.c_int, [_P, _I64, _I32, _P, _I32, _I32, _P, _I64, _P, _I64, _P]),
    "moe_norm_weight": (C.c_int, [_P, _I32, _P, _P]),
    "moe_choose_block_m": (C.c_int, [_I64, _I32, _I64, _I32, C.POINTER(_I32)]),
    "moe_gemm_choose": (C.c_int, [C.POINTER(MoeWeights), _I64, _I32, _I32, C.POINTER(MoeGemmConfig)]),
    "moe_gemm_choose_occ": (C.c_int, [C.POINTER(MoeWeights), _I64, _I32, _I32, C.POINTER(_I32 * 3),
                                      C.POINTER(MoeGemmConfig)]),
    "moe_gemm_occupancy": (C.c_int, [C.POINTER(MoeWeights), _I32, _I32, C.POINTER(_I32 * 3)]),
    "moe_w4a16_gemm": (C.c_int, [_P, _I64, _I32, _P, _I32, C.POINTER(MoeWeights), _P, _P, _P,
                                 _I64, _I32, _I32, C.POINTER(MoeGemmConfig), _P]),
    "moe_w4a16_gemm_act": (C.c_int, [C.c_int, _F, _F, _P, _I64, _I32, _P, _I32, C.POINTER(MoeWeights), _P,
                                     _P, _P, _I64, _I32, _I32, C.POINTER(MoeGemmConfig), _P]),
    "moe_w4a16_gemm_act_routed": (C.c_int, [C.c_int, _F, _F, _P, _I64, _I32, _P, _I32, C.POINTER(MoeWeights),
                                            _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P,
                                            C.POINTER(MoeGemmConfig), _P]),
    "moe_act": (C.c_int, [C.c_int, _P, _I32, _P, _I32, _I64, _I32, _P, _F, _F, _P]),
    "moe_combine": (C.c_int, [_P, _P, _P, _P, _F, _F, _I64, _I32, _I32, _P, _P]),
    "moe_w4a16_gemm_combine": (C.c_int, [_P, _I64, _I32, _P, _I32, C.POINTER(MoeWeights), _P, _P, _P,
                                         _I64, _I32, _I32, _P, _P, _F, _P, _I64, _P, _I32,
                                         C.POINTER(MoeGemmConfig), _P]),
    "moe_w4a16_gemm_combine_noalloc": (C.c_int, [_P, _I64, _I32, _P, _I32, C.POINTER(MoeWeights), _P, _P, _P,
                                                 _I64, _I32, _I32, _P, _P, _F, _P, _I32,
                                                 C.POINTER(MoeGemmConfig), _P]),
    "moe_fp8_requant_choose": (C.c_int, [_I32, _I32, _I32, _I32, _I32, C.POINTER(MoeRequantConfig)]),
    "moe_fp8_requant": (C.c_int, [_P, _P, _I64, _I64, _I64, _P, _P, _I32, _I32, _I32, _I32, _P,
                                  C.POINTER(MoeRequantConfig), _P]),
}

_lib = None


def lib():
    """The loaded library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m quantized_mixture_experts_align_amd.build`"
                " (there is no fallback implementation)")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def check(rc: int, what: str = "") -> None:
    if rc == MOE_OK:
        return
    msg = lib().moe_last_error().decode(errors="replace")
    text = f"{what}: {msg} (status {rc})" if what else f"{msg} (status {rc})"
    if rc in (MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ESIZE):
        raise ValueError(text)
    raise MoeError(text)
