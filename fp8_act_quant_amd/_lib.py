"""ctypes loader for libfp8q.so (the C ABI in include/fp8q.h).

Argument marshalling only: every step of the quantisation and GEMM runs in the HIP
kernels behind this library. If the library is missing the import fails; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

FP8Q_OK = 0
FP8Q_ERR_NULL = 1
FP8Q_ERR_SHAPE = 2
FP8Q_ERR_ALIGN = 3
FP8Q_ERR_DTYPE = 4
FP8Q_ERR_UNSUPPORTED = 5
FP8Q_ERR_LAUNCH = 6
FP8Q_ERR_WORKSPACE = 7
FP8Q_NOALLOC_SCRATCH_BYTES = 32 << 20

FP8Q_OUT_F32 = 0
FP8Q_OUT_BF16 = 1
FP8Q_GEMM_FP8_PRODUCTS = 0x100
FP8Q_GEMM_EXACT_SLICES = 0x200
FP8Q_SA_KMAJOR = 0x1000

# name -> (restype, argtypes); the exports of include/fp8q.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "fp8_act_quant": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_act_quant_kmajor": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_weight_quant": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_weight_dequant": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_block_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P,
                                      ctypes.c_size_t, _P]),
    "fp8_block_gemm_bias": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P,
                                           ctypes.c_size_t, _P]),
    "fp8_block_gemm_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, ctypes.c_int]),
    "fp8_block_gemm_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P]),
    "fp8_bf16_gemm": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P]),
    "fp8_grouped_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _P]),
    "fp8_act_quant_t": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_weight_transpose": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _P]),
    "fp8_rowwise_gemm": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "fp8_rowwise_gemm_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, ctypes.c_int]),
    "fp8q_gemm_force_config": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "fp8q_gemm_config_name": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8q_gemm_plan": (ctypes.c_int, [_I64, _I64, _I64, ctypes.c_int, _P, _P]),
    "fp8q_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8q_version": (ctypes.c_int, []),
}


class Fp8qError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc --offload-arch=gfx950); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.fp8q_strerror(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != FP8Q_OK:
        raise Fp8qError(fn, status, strerror(status))
