"""CPU oracle for FP8 (E4M3) block quantisation and the block-scaled GEMM.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The GPU library never
imports it and shares no code with it; the product path fails loudly if its own
HIP library is missing instead of falling back to anything here.

The arithmetic lives in ``fp8_oracle.c`` (plain C, gcc, IEEE fp32/fp64, no
fast-math); this module only marshals numpy arrays through ctypes. Pages and
sections followed are cited in that file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BLOCK = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = [
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    sig = {
        "or_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "or_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "or_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
        "or_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "or_act_quant": (None, [P, P, P, I64, I64]),
        "or_weight_quant": (None, [P, P, P, I64, I64]),
        "or_weight_dequant": (None, [P, P, P, I64, I64]),
        "or_block_gemm": (None, [P, P, P, P, I64, I64, I64, P, P]),
        "or_block_gemm_sampled": (None, [P, P, P, P, I64, I64, I64, P, P, I64, P, P]),
        "or_matmul_bf16_sampled": (None, [P, P, I64, P, P, I64, P]),
        "or_matmul_bf16": (None, [P, P, I64, I64, I64, P, P]),
        "or_rowwise_gemm": (None, [P, P, P, P, I64, I64, I64, P, P]),
        "or_rowwise_gemm_sampled": (None, [P, P, P, P, I64, P, P, I64, P, P]),
        "or_e4m3_encode_batch": (None, [P, P, I64]),
        "or_f32_to_bf16_batch": (None, [P, P, I64]),
        "or_f64_to_bf16_batch": (None, [P, P, I64]),
        "or_num_threads": (ctypes.c_int, []),
        "or_set_num_threads": (None, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


# ----------------------------------------------------------------------------- scalars

def e4m3_decode(code: int) -> float:
    """Closed-form OCP E4M3FN decode of one code (NaN for 0x7F / 0xFF)."""
    return _load().or_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(value: float) -> int:
    """E4M3 round-to-nearest-even with saturation of one fp32 value."""
    return int(_load().or_e4m3_encode(float(np.float32(value))))


def e4m3_decode_all() -> np.ndarray:
    """Decoded value of every code 0..255 as float64 (NaN for the two NaN codes)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = _c(v.astype(np.float32, copy=False), np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().or_e4m3_encode_batch(_ptr(v), _ptr(out), v.size)
    return out


def f32_to_bf16_array(v: np.ndarray) -> np.ndarray:
    v = _c(v.astype(np.float32, copy=False), np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().or_f32_to_bf16_batch(_ptr(v), _ptr(out), v.size)
    return out


def f64_to_bf16_array(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 bit patterns (nearest, ties to even)."""
    v = _c(v.astype(np.float64, copy=False), np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().or_f64_to_bf16_batch(_ptr(v), _ptr(out), v.size)
    return out


def bf16_to_f32_array(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- path

def act_quant(x_bf16: np.ndarray):
    """x: uint16 (bf16 bits) [M, K] -> (q uint8 [M, K], s float32 [M, K/128])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // BLOCK), dtype=np.float32)
    _load().or_act_quant(_ptr(x), _ptr(q), _ptr(s), M, K)
    return q, s


def weight_quant(w_bf16: np.ndarray):
    """w: uint16 [N, K] -> (q uint8 [N, K], s float32 [ceil(N/128), K/128])."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty(((N + BLOCK - 1) // BLOCK, K // BLOCK), dtype=np.float32)
    _load().or_weight_quant(_ptr(w), _ptr(q), _ptr(s), N, K)
    return q, s


def act_quant_t(x_bf16: np.ndarray):
    """Token-wise quantisation for the weight gradient (the 1x128 activation rule applied
    along the token dimension): x uint16 (bf16 bits) [M, C] -> (qt uint8 [C, ldq],
    st float32 [C, ldq/128]), ldq = ceil(M/128)*128. The tokens are zero-padded to ldq and
    the transposed matrix goes through act_quant (a zero token enters no amax and encodes to
    code 0)."""
    x = _c(x_bf16, np.uint16)
    M, C = x.shape
    ldq = -(-M // BLOCK) * BLOCK
    xt = np.zeros((C, ldq), dtype=np.uint16)
    xt[:, :M] = x.T
    return act_quant(xt)


def weight_transpose(q: np.ndarray, s: np.ndarray):
    """Wq [N, K] -> Wq^T [K, N]; scale grid [ceil(N/128), K/128] -> its transpose."""
    return np.ascontiguousarray(np.asarray(q, dtype=np.uint8).T), np.ascontiguousarray(np.asarray(s, np.float32).T)


def weight_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """q: uint8 [N, K], s: float32 [ceil(N/128), K/128] -> uint16 (bf16 bits) [N, K]."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    N, K = q.shape
    if s.shape != ((N + BLOCK - 1) // BLOCK, K // BLOCK):
        raise ValueError("scale grid shape mismatch")
    w = np.empty((N, K), dtype=np.uint16)
    _load().or_weight_dequant(_ptr(q), _ptr(s), _ptr(w), N, K)
    return w


def block_gemm(aq, sa, wq, sw):
    """Full float64 result and bound: (y [M, N], bound [M, N])."""
    aq = _c(aq, np.uint8)
    wq = _c(wq, np.uint8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    M, K = aq.shape
    N = wq.shape[0]
    _check_gemm_shapes(aq, sa, wq, sw)
    y = np.empty((M, N), dtype=np.float64)
    b = np.empty((M, N), dtype=np.float64)
    _load().or_block_gemm(_ptr(aq), _ptr(sa), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), _ptr(b))
    return y, b


def block_gemm_sampled(aq, sa, wq, sw, rows, cols):
    """float64 result and bound at outputs (rows[i], cols[i])."""
    aq = _c(aq, np.uint8)
    wq = _c(wq, np.uint8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    _check_gemm_shapes(aq, sa, wq, sw)
    M, K = aq.shape
    N = wq.shape[0]
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows/cols mismatch")
    if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
        raise ValueError("sample index out of range")
    y = np.empty(rows.shape, dtype=np.float64)
    b = np.empty(rows.shape, dtype=np.float64)
    _load().or_block_gemm_sampled(_ptr(aq), _ptr(sa), _ptr(wq), _ptr(sw), M, N, K,
                                  _ptr(rows), _ptr(cols), rows.size, _ptr(y), _ptr(b))
    return y, b


def grouped_gemm_sampled(aq, sa, wq, sw, offsets, rows, cols):
    """Routed-expert GEMM at outputs (rows[i], cols[i]): row r belongs to the expert e with
    offsets[e] <= r < offsets[e+1] and is that expert's block-scaled GEMM row (the
    composition of block_gemm_sampled over experts; wq [E, N, K], sw [E, ceil(N/128), K/128]).
    Returns (float64 result, bound)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    y = np.full(rows.shape, np.nan)
    b = np.full(rows.shape, np.nan)
    expert = np.searchsorted(offsets, rows, side="right") - 1
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        r0 = offsets[e]
        ye, be = block_gemm_sampled(aq[r0:offsets[e + 1]], sa[r0:offsets[e + 1]], wq[e], sw[e],
                                    rows[sel] - r0, cols[sel])
        y[sel] = ye
        b[sel] = be
    return y, b


def grouped_gemm(aq, sa, wq, sw, offsets):
    """Routed-expert GEMM, every output (rows owned by no expert are NaN)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    R = aq.shape[0]
    N = wq.shape[1]
    y = np.full((R, N), np.nan)
    b = np.full((R, N), np.nan)
    for e in range(wq.shape[0]):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            y[r0:r1], b[r0:r1] = block_gemm(aq[r0:r1], sa[r0:r1], wq[e], sw[e])
    return y, b


def rowwise_gemm(aq, sa, bq, sb):
    """GEMM with per-row scales on both operands (sb [N, K/128]): full float64 result and
    bound (y [M, N], bound [M, N])."""
    aq, bq = _c(aq, np.uint8), _c(bq, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    M, K = aq.shape
    N = bq.shape[0]
    if bq.shape[1] != K or K % BLOCK or sa.shape != (M, K // BLOCK) or sb.shape != (N, K // BLOCK):
        raise ValueError("shape mismatch")
    y = np.empty((M, N), dtype=np.float64)
    b = np.empty((M, N), dtype=np.float64)
    _load().or_rowwise_gemm(_ptr(aq), _ptr(sa), _ptr(bq), _ptr(sb), M, N, K, _ptr(y), _ptr(b))
    return y, b


def rowwise_gemm_sampled(aq, sa, bq, sb, rows, cols):
    """rowwise_gemm at outputs (rows[i], cols[i])."""
    aq, bq = _c(aq, np.uint8), _c(bq, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    M, K = aq.shape
    N = bq.shape[0]
    if bq.shape[1] != K or K % BLOCK or sa.shape != (M, K // BLOCK) or sb.shape != (N, K // BLOCK):
        raise ValueError("shape mismatch")
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    if rows.shape != cols.shape or (rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0
                                                   or cols.max() >= N)):
        raise ValueError("bad sample coordinates")
    y = np.empty(rows.shape, dtype=np.float64)
    b = np.empty(rows.shape, dtype=np.float64)
    _load().or_rowwise_gemm_sampled(_ptr(aq), _ptr(sa), _ptr(bq), _ptr(sb), K, _ptr(rows), _ptr(cols), rows.size,
                                    _ptr(y), _ptr(b))
    return y, b


def matmul_bf16(x_bf16, w_bf16):
    """The bf16 linear of the linear() listing's bf16 branch, y = x . w^T over bf16 values
    (x [M, K], w [N, K] as uint16 bit patterns), in float64: (y [M, N], bound [M, N]) with
    bound = sum_k |x_k w_k|."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("K mismatch")
    y = np.empty((M, N), dtype=np.float64)
    b = np.empty((M, N), dtype=np.float64)
    _load().or_matmul_bf16(_ptr(x), _ptr(w), M, N, K, _ptr(y), _ptr(b))
    return y, b


def matmul_bf16_sampled(x_bf16, w_bf16, rows, cols):
    """Unquantised float64 x . w^T at sampled outputs (information only)."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    K = x.shape[1]
    if w.shape[1] != K:
        raise ValueError("K mismatch")
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    y = np.empty(rows.shape, dtype=np.float64)
    _load().or_matmul_bf16_sampled(_ptr(x), _ptr(w), K, _ptr(rows), _ptr(cols), rows.size,
                                   _ptr(y))
    return y


def _check_gemm_shapes(aq, sa, wq, sw):
    M, K = aq.shape
    N, K2 = wq.shape
    if K != K2 or K % BLOCK:
        raise ValueError("K mismatch or not a multiple of 128")
    if sa.shape != (M, K // BLOCK):
        raise ValueError("activation scale shape mismatch")
    if sw.shape != ((N + BLOCK - 1) // BLOCK, K // BLOCK):
        raise ValueError("weight scale shape mismatch")


def num_threads() -> int:
    return int(_load().or_num_threads())


def set_num_threads(n: int) -> None:
    _load().or_set_num_threads(int(n))
