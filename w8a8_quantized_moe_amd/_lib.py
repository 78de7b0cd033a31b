"""ctypes loader for libw8a8moe.so (argument marshalling only).

The library is built in-tree by ``w8a8_quantized_moe_amd.build``.  If it is
missing this module raises at import time: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch must be loaded first: it brings its own copy of the HIP runtime
# (requested as libamdhip64.so), and the library's dependency on
# libamdhip64.so.7 then resolves to that same copy by soname.  Loading the
# library first would map the system runtime as well, and two runtimes in one
# process do not share devices, streams or memory.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw8a8moe.so")

W8A8_OK = 0
W8A8_ERR_INVALID_ARGUMENT = 1
W8A8_ERR_UNSUPPORTED_SHAPE = 2
W8A8_ERR_WORKSPACE_TOO_SMALL = 3
W8A8_ERR_MISALIGNED = 4
W8A8_ERR_HIP = 5

CODE_INT8 = 0
CODE_FP8 = 1       # E4M3 codes, exact products summed in fp32
CODE_FP8_FAST = 2  # E4M3 codes on the FP8 matrix cores (products aligned per 8-k group)
PACK_PLAIN = 0
PACK_GATE_UP = 1


class W8A8Error(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("E", ctypes.c_int64),
                ("top_k", ctypes.c_int64), ("I", ctypes.c_int64)]


SCALE_DYNAMIC, SCALE_CLIPPED, SCALE_STATIC = 0, 1, 2
SCALE_COL_RECIPROCAL = 0x10  # or'ed into the mode: the column factor is applied as 1/col_mul


class MoeWeights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("w_gate_up", ctypes.c_void_p), ("s_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("s_down", ctypes.c_void_p), ("code", ctypes.c_int32),
                ("x_smooth", ctypes.c_void_p), ("x_scale_mode", ctypes.c_int32),
                ("x_clip", ctypes.c_float)]


LAYOUT_FIELDS = ["total_bytes", "x_q", "x_scale", "logits", "topk_ids", "topk_w", "expert_counts",
                 "expert_offsets", "sorted_assign", "h", "h_q", "h_scale", "o", "internal"]


class MoeLayout(ctypes.Structure):
    _fields_ = [(f, ctypes.c_size_t) for f in LAYOUT_FIELDS]


# exported symbol -> (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "w8a8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w8a8_last_error": (ctypes.c_char_p, []),
    "w8a8_abi_version": (ctypes.c_int, []),
    "w8a8_quantize_rows": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "w8a8_quantize_rows_fp8": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "w8a8_quantize_rows_ex": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, ctypes.c_int32, ctypes.c_float,
                                             ctypes.c_int32, _P, _P, _P]),
    "w8a8_gemm_fp8": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_gemm_fp8_fast": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_pack_weights_size": (ctypes.c_int, [_I64, _I64, _I64, ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_size_t)]),
    "w8a8_pack_weights": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_int, _P, _P]),
    "w8a8_gemm": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_gemm_i32": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_moe_workspace_query": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeLayout)]),
    "w8a8_moe_forward": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _P, _P,
                                        _P, ctypes.c_size_t, _P]),
    "w8a8_moe_forward_events": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights),
                                               _P, _P, _P, ctypes.c_size_t, _P, _P]),
    "w8a8_moe_gate_up_acc": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _P,
                                            ctypes.c_size_t, _P, _P]),
    "w8a8_moe_forward_static": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _P, _P,
                                               _P]),
    "w8a8_moe_forward_fused": (ctypes.c_int, [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _P, _P,
                                              _P, ctypes.c_size_t, _P]),
}

FUSED_MAX_T = 64  # the single-launch layer's token limit

STATIC_WORKSPACE_BYTES = 64 << 20  # W8A8_STATIC_WORKSPACE_BYTES

MOE_STAGES = ["quant", "route", "gate_up", "requant", "down", "combine"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libw8a8moe.so not found at {LIB_PATH}; build it with "
            "`python w8a8_quantized_moe_amd/build.py` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def check(status: int) -> None:
    if status != W8A8_OK:
        name = lib.w8a8_status_string(status).decode()
        detail = lib.w8a8_last_error().decode()
        raise W8A8Error(status, name, detail)
