"""FP8 (E4M3) fine-grained block quantisation and block-scaled GEMM for AMD MI355X.

Python names follow the linear() listing on the pomoai.com "DeepSeek-V3" page (FP8
mixed-precision training section): ``act_quant(x, block_size) -> (x_fp8, scale)``,
``fp8_gemm(x, scale, weight, weight_scale) -> y`` and ``weight_dequant(weight,
weight_scale)``, plus the weight quantiser that produces the 128x128-block format.

This module only marshals arguments: it checks dtypes, shapes and devices, allocates
the outputs with torch and calls the C ABI of libfp8q.so on torch's current HIP
stream. Every arithmetic step runs in the gfx950 kernels behind that library.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import (FP8Q_GEMM_EXACT_SLICES, FP8Q_GEMM_FP8_PRODUCTS, FP8Q_OUT_BF16, FP8Q_OUT_F32, FP8Q_SA_KMAJOR,
                   Fp8qError, check, lib)

BLOCK = 128

__all__ = [
    "BLOCK", "Fp8qError", "act_quant", "weight_quant", "weight_dequant", "fp8_gemm", "fp8_grouped_gemm",
    "linear", "gemm_workspace_bytes", "lib", "act_quant_t", "weight_transpose", "fp8_gemm_rowwise",
    "linear_backward", "bf16_gemm",
]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, align: int = 16) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() and t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")


# K-block-major activation scales are limited to this many (32-bit byte offsets in the GEMM)
MAX_KMAJOR_SCALES = 1 << 29


def act_quant(x: torch.Tensor, block_size: int = BLOCK, scale_layout: str = "row"):
    """Per-token, per-128-channel quantisation of a bf16 activation [..., K].

    Returns ``(q, s)``: q float8_e4m3fn [..., K], s float32 [..., K/128]. With
    scale_layout="kmajor" s has the same shape and values but K-block-major storage
    (``s.movedim(-1, 0)`` is contiguous), the layout in which fp8_gemm reads one K slice's
    scales as contiguous bytes; it needs fewer than 2^29 scales."""
    if block_size != BLOCK:
        raise ValueError("only block_size=128 is supported")
    if scale_layout not in ("row", "kmajor"):
        raise ValueError('scale_layout must be "row" or "kmajor"')
    _need(x, "x", torch.bfloat16)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("the last dimension must be a multiple of 128")
    M = math.prod(x.shape[:-1])
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    with torch.cuda.device(x.device):
        if scale_layout == "row":
            s = torch.empty((*x.shape[:-1], K // BLOCK), dtype=torch.float32, device=x.device)
            check("fp8_act_quant", lib.fp8_act_quant(x.data_ptr(), q.data_ptr(), s.data_ptr(), M, K,
                                                     _stream(x)))
        else:
            st = torch.empty((K // BLOCK, *x.shape[:-1]), dtype=torch.float32, device=x.device)
            check("fp8_act_quant_kmajor", lib.fp8_act_quant_kmajor(x.data_ptr(), q.data_ptr(), st.data_ptr(), M, K,
                                                                   _stream(x)))
            s = st.movedim(0, -1)
    return q, s


def weight_quant(w: torch.Tensor):
    """128x128 block quantisation of a bf16 weight [N, K].

    Returns ``(q, s)``: q float8_e4m3fn [N, K], s float32 [ceil(N/128), K/128]."""
    _need(w, "w", torch.bfloat16)
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    q = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=w.device)
    s = torch.empty(((N + BLOCK - 1) // BLOCK, K // BLOCK), dtype=torch.float32, device=w.device)
    with torch.cuda.device(w.device):
        check("fp8_weight_quant", lib.fp8_weight_quant(w.data_ptr(), q.data_ptr(), s.data_ptr(), N, K,
                                                       _stream(w)))
    return q, s


def weight_dequant(q: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    """bf16 weight [N, K] from its E4M3 codes and 128x128 block scales."""
    _need(q, "q", torch.float8_e4m3fn)
    _need(s, "s", torch.float32, align=4)
    if q.dim() != 2:
        raise ValueError("q must be 2-D [N, K]")
    N, K = q.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    if tuple(s.shape) != ((N + BLOCK - 1) // BLOCK, K // BLOCK):
        raise ValueError(f"s must be [{(N + BLOCK - 1) // BLOCK}, {K // BLOCK}]")
    w = torch.empty((N, K), dtype=torch.bfloat16, device=q.device)
    with torch.cuda.device(q.device):
        check("fp8_weight_dequant", lib.fp8_weight_dequant(q.data_ptr(), s.data_ptr(), w.data_ptr(), N, K,
                                                           _stream(q)))
    return w


_MODES = {"default": 0, "fp8": FP8Q_GEMM_FP8_PRODUCTS, "exact": FP8Q_GEMM_EXACT_SLICES}


def _gemm_code(out_dtype, mode: str) -> int:
    return (FP8Q_OUT_BF16 if out_dtype == torch.bfloat16 else FP8Q_OUT_F32) | _MODES[mode]


def gemm_workspace_bytes(M: int, N: int, K: int, out_dtype=torch.bfloat16, mode: str = "default") -> int:
    """Bytes of workspace that let fp8_gemm use its split-K schedule for this shape (0 if
    the shape does not use one)."""
    return int(lib.fp8_block_gemm_workspace_bytes(M, N, K, _gemm_code(out_dtype, mode)))


# Split-K workspaces kept per (device, stream) and reused by every call (the library needs
# no initialised contents). One per stream, because calls that may overlap must not share one.
_WORKSPACES: dict = {}


def _auto_workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def _scale_layout(a_s: torch.Tensor) -> bool:
    """True for K-block-major activation scales (a_s.movedim(-1, 0) contiguous), False for
    row-major ones; where both hold (one row or one K slice) the two layouts coincide."""
    if not isinstance(a_s, torch.Tensor):
        raise TypeError("a_s must be a torch.Tensor")
    if a_s.device.type != "cuda":
        raise ValueError("a_s must be a GPU tensor")
    if a_s.dtype != torch.float32:
        raise TypeError(f"a_s must be torch.float32, got {a_s.dtype}")
    if a_s.numel() and a_s.data_ptr() % 4:
        raise ValueError("a_s must be 4-byte aligned")
    if a_s.is_contiguous():
        return False
    if a_s.dim() >= 2 and a_s.movedim(-1, 0).is_contiguous():
        return True
    raise ValueError("a_s must be contiguous or K-block-major (a_s.movedim(-1, 0) contiguous)")


def fp8_gemm(a: torch.Tensor, a_s: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor,
             out_dtype=torch.bfloat16, workspace="auto", out: torch.Tensor | None = None,
             mode: str = "default", bias: torch.Tensor | None = None) -> torch.Tensor:
    """Block-scaled Y = A . W^T. a: float8_e4m3fn [..., K] with scales [..., K/128]
    (contiguous, or K-block-major as act_quant(..., scale_layout="kmajor") returns them);
    w: float8_e4m3fn [N, K] with scales [ceil(N/128), K/128]. Returns [..., N] in
    out_dtype (torch.float32 or torch.bfloat16).

    mode: "fp8" forms every 128-wide slice partial on the FP8 matrix unit, "exact" on the
    f16 matrix unit from exactly converted operands; "default" is "exact" for float32
    output and "fp8" for bfloat16 output.

    workspace: "auto" (a workspace cached per device and stream), None (no split-K), or a
    uint8 tensor of any contents.

    bias: optional [N] vector, added in fp32 to every row before the output rounding."""
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    _need(a, "a", torch.float8_e4m3fn)
    _need(w, "w", torch.float8_e4m3fn)
    sa_kmajor = _scale_layout(a_s)
    _need(w_s, "w_s", torch.float32, align=4)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    K = a.shape[-1]
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError("w must be [N, K] with the activation's K")
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    N = w.shape[0]
    M = math.prod(a.shape[:-1])
    if tuple(a_s.shape) != (*a.shape[:-1], K // BLOCK):
        raise ValueError("a_s must be [..., K/128]")
    if tuple(w_s.shape) != ((N + BLOCK - 1) // BLOCK, K // BLOCK):
        raise ValueError("w_s must be [ceil(N/128), K/128]")
    shape = (*a.shape[:-1], N)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=a.device)
    else:
        _need(out, "out", out_dtype)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {shape}")
    code = _gemm_code(out_dtype, mode) | (FP8Q_SA_KMAJOR if sa_kmajor else 0)
    ws_ptr, ws_bytes = 0, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a tensor')
        need = int(lib.fp8_block_gemm_workspace_bytes(M, N, K, code)) if M and N and K else 0
        if need:
            ws = _auto_workspace(a.device, _stream(a), need)
            ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    elif workspace is not None:
        _need(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    b_ptr = None
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.device != a.device or tuple(bias.shape) != (N,):
            raise ValueError(f"bias must be a [{N}] tensor on {a.device}")
        bias = bias.to(torch.float32).contiguous()
        b_ptr = bias.data_ptr()
    with torch.cuda.device(a.device):
        check("fp8_block_gemm_bias", lib.fp8_block_gemm_bias(a.data_ptr(), a_s.data_ptr(), w.data_ptr(),
                                                             w_s.data_ptr(), b_ptr, out.data_ptr(), code, M, N, K,
                                                             ws_ptr or None, ws_bytes, _stream(a)))
    return out


def fp8_grouped_gemm(a: torch.Tensor, a_s: torch.Tensor, w: torch.Tensor, w_s: torch.Tensor,
                     offsets: torch.Tensor, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                     mode: str = "default") -> torch.Tensor:
    """Routed-expert block-scaled GEMM in one launch. a: float8_e4m3fn [rows, K] with scales
    [rows, K/128], the rows of expert e being offsets[e] .. offsets[e+1]-1; w: float8_e4m3fn
    [E, N, K] with scales [E, ceil(N/128), K/128]; offsets: int64 [E + 1] on the device,
    non-decreasing from 0 to rows. Returns [rows, N]: row r is a[r] times the weight of the
    expert that owns it. Rows owned by no expert (offsets not reaching rows) are left as
    they were in `out`, or uninitialised. mode as for fp8_gemm; no split-K."""
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    _need(a, "a", torch.float8_e4m3fn)
    _need(w, "w", torch.float8_e4m3fn)
    _need(a_s, "a_s", torch.float32, align=4)
    _need(w_s, "w_s", torch.float32, align=4)
    _need(offsets, "offsets", torch.int64, align=8)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if a.dim() != 2 or w.dim() != 3:
        raise ValueError("a must be [rows, K] and w [E, N, K]")
    rows, K = a.shape
    E, N = w.shape[0], w.shape[1]
    if w.shape[2] != K:
        raise ValueError("w must be [E, N, K] with the activation's K")
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    if tuple(a_s.shape) != (rows, K // BLOCK):
        raise ValueError("a_s must be [rows, K/128]")
    if tuple(w_s.shape) != (E, (N + BLOCK - 1) // BLOCK, K // BLOCK):
        raise ValueError("w_s must be [E, ceil(N/128), K/128]")
    if tuple(offsets.shape) != (E + 1,):
        raise ValueError("offsets must be [E + 1]")
    if offsets.device != a.device:
        raise ValueError("offsets must be on the activation's device")
    shape = (rows, N)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=a.device)
    else:
        _need(out, "out", out_dtype)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {shape}")
    with torch.cuda.device(a.device):
        check("fp8_grouped_gemm", lib.fp8_grouped_gemm(a.data_ptr(), a_s.data_ptr(), w.data_ptr(), w_s.data_ptr(),
                                                       offsets.data_ptr(), out.data_ptr(), _gemm_code(out_dtype, mode),
                                                       E, rows, N, K, _stream(a)))
    return out


def bf16_gemm(x: torch.Tensor, w: torch.Tensor, bias: torch.Tensor | None = None,
              out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = x . w^T (+ bias) on bf16 operands, fp32 accumulation: the bf16 GEMM of linear()'s
    bf16 branch. x: bfloat16 [..., K]; w: bfloat16 [N, K] (K a multiple of 64); bias:
    optional [N], added in fp32 before the output rounding. Returns [..., N] in out_dtype
    (torch.bfloat16 or torch.float32)."""
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.bfloat16)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    K = x.shape[-1]
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError("w must be [N, K] with the activation's K")
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    N = w.shape[0]
    M = math.prod(x.shape[:-1])
    shape = (*x.shape[:-1], N)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=x.device)
    else:
        _need(out, "out", out_dtype, align=4)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {shape}")
    b_ptr = None
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.device != x.device or tuple(bias.shape) != (N,):
            raise ValueError(f"bias must be a [{N}] tensor on {x.device}")
        bias = bias.to(torch.float32).contiguous()
        b_ptr = bias.data_ptr()
    code = FP8Q_OUT_BF16 if out_dtype == torch.bfloat16 else FP8Q_OUT_F32
    with torch.cuda.device(x.device):
        check("fp8_bf16_gemm", lib.fp8_bf16_gemm(x.data_ptr(), w.data_ptr(), b_ptr, out.data_ptr(), code, M, N, K,
                                                 _stream(x)))
    return out


def linear(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor | None = None,
           weight_scale: torch.Tensor | None = None, gemm_impl: str = "fp8",
           out_dtype=torch.bfloat16) -> torch.Tensor:
    """y = x . weight^T (+ bias) for bf16 activations x [..., K], as the pomoai.com
    "DeepSeek-V3" page's linear() describes it (FP8 mixed-precision training section), with
    every product in this library's kernels:

    * a weight stored unquantised (bfloat16 [N, K]) goes through the bf16 GEMM;
    * an FP8 weight (float8_e4m3fn [N, K] with weight_scale [ceil(N/128), K/128]) with
      gemm_impl "bf16" is dequantised by weight_dequant and then goes through the bf16 GEMM;
    * an FP8 weight with gemm_impl "fp8" (the default): x is quantised by act_quant
      (K-block-major scales) and multiplied by the block-scaled GEMM, the bias added in its
      epilogue.

    Other weight dtypes are rejected. bias: optional [N]."""
    if gemm_impl not in ("fp8", "bf16"):
        raise ValueError('gemm_impl must be "fp8" or "bf16"')
    if weight.dtype == torch.bfloat16:
        return bf16_gemm(x, weight, bias, out_dtype=out_dtype)
    if weight.dtype != torch.float8_e4m3fn:
        raise TypeError(f"weight must be torch.float8_e4m3fn (with weight_scale) or torch.bfloat16, got {weight.dtype}")
    if weight_scale is None:
        raise ValueError("an FP8 weight needs its weight_scale")
    if gemm_impl == "bf16":
        return bf16_gemm(x, weight_dequant(weight, weight_scale), bias, out_dtype=out_dtype)
    # K-block-major scales: the GEMM fetches each K slice's scales as whole cache lines
    M, nkb = math.prod(x.shape[:-1]), x.shape[-1] // BLOCK
    q, s = act_quant(x, scale_layout="kmajor" if M * nkb < MAX_KMAJOR_SCALES else "row")
    return fp8_gemm(q, s, weight, weight_scale, out_dtype=out_dtype, bias=bias)


# ---------------------------------------------------------------------------------------
# Training GEMMs (backward of y = x W^T): see include/fp8q.h for the quantisation reading.

def act_quant_t(x: torch.Tensor):
    """Token-wise quantisation of a bf16 [M, C] tensor (C a multiple of 8), transposed:
    returns ``(qt, st)``, qt float8_e4m3fn [C, ldq] and st float32 [C, ldq/128] with
    ldq = ceil(M/128)*128; tokens past M are code 0."""
    _need(x, "x", torch.bfloat16)
    if x.dim() != 2:
        raise ValueError("x must be [M, C]")
    M, C = x.shape
    if C % 8:
        raise ValueError("C must be a multiple of 8")
    ldq = -(-M // BLOCK) * BLOCK
    qt = torch.empty((C, ldq), dtype=torch.float8_e4m3fn, device=x.device)
    st = torch.empty((C, ldq // BLOCK), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        check("fp8_act_quant_t", lib.fp8_act_quant_t(x.data_ptr(), qt.data_ptr(), st.data_ptr(), M, C, _stream(x)))
    return qt, st


def weight_transpose(q: torch.Tensor, s: torch.Tensor):
    """FP8 weight [N, K] and its block scales [ceil(N/128), K/128] -> the transposed weight
    [K, N] and scales [K/128, ceil(N/128)] (the same codes and block scales)."""
    _need(q, "q", torch.float8_e4m3fn)
    _need(s, "s", torch.float32, align=4)
    N, K = q.shape
    if K % BLOCK or tuple(s.shape) != ((N + BLOCK - 1) // BLOCK, K // BLOCK):
        raise ValueError("q must be [N, K] (K a multiple of 128) with scales [ceil(N/128), K/128]")
    qt = torch.empty((K, N), dtype=torch.float8_e4m3fn, device=q.device)
    st = torch.empty((K // BLOCK, (N + BLOCK - 1) // BLOCK), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        check("fp8_weight_transpose", lib.fp8_weight_transpose(q.data_ptr(), s.data_ptr(), qt.data_ptr(),
                                                               st.data_ptr(), N, K, _stream(q)))
    return qt, st


def fp8_gemm_rowwise(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                     out_dtype=torch.float32, workspace="auto", out: torch.Tensor | None = None,
                     mode: str = "default") -> torch.Tensor:
    """Y [M, N] = A . B^T with per-row scales on both operands: a float8_e4m3fn [M, K] with
    scales [M, K/128], b float8_e4m3fn [N, K] with scales [N, K/128]. mode and workspace as
    for fp8_gemm."""
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    for t, n, dt, al in ((a, "a", torch.float8_e4m3fn, 16), (b, "b", torch.float8_e4m3fn, 16),
                         (a_s, "a_s", torch.float32, 4), (b_s, "b_s", torch.float32, 4)):
        _need(t, n, dt, align=al)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1] or a.shape[1] % BLOCK:
        raise ValueError("a [M, K] and b [N, K] with K a multiple of 128")
    M, K = a.shape
    N = b.shape[0]
    if tuple(a_s.shape) != (M, K // BLOCK) or tuple(b_s.shape) != (N, K // BLOCK):
        raise ValueError("a_s must be [M, K/128] and b_s [N, K/128]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    else:
        _need(out, "out", out_dtype)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be {(M, N)}")
    code = _gemm_code(out_dtype, mode)
    ws_ptr, ws_bytes = 0, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a tensor')
        need = int(lib.fp8_rowwise_gemm_workspace_bytes(M, N, K, code)) if M and N and K else 0
        if need:
            ws = _auto_workspace(a.device, _stream(a), need)
            ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    elif workspace is not None:
        _need(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(a.device):
        check("fp8_rowwise_gemm", lib.fp8_rowwise_gemm(a.data_ptr(), a_s.data_ptr(), b.data_ptr(), b_s.data_ptr(),
                                                       out.data_ptr(), code, M, N, K, ws_ptr or None, ws_bytes,
                                                       _stream(a)))
    return out


def linear_backward(dy: torch.Tensor, x: torch.Tensor, weight: torch.Tensor, weight_scale: torch.Tensor,
                    weight_t=None, dx_dtype=torch.bfloat16, dw_dtype=torch.float32):
    """FP8 backward of y = x W^T (W an FP8 weight [N, K] with 128x128 block scales):
    dx [M, K] = dY . W (dY quantised 1x128 along N; N a multiple of 128) and
    dW [N, K] = dY^T . X (both quantised 1x128 along the tokens). weight_t: optional
    (W^T codes, scales) from weight_transpose, reused across steps. Returns (dx, dw)."""
    if dy.dim() != 2 or x.dim() != 2 or dy.shape[0] != x.shape[0]:
        raise ValueError("dy [M, N] and x [M, K]")
    if weight_t is None:
        weight_t = weight_transpose(weight, weight_scale)
    dyq, sdy = act_quant(dy)
    dx = fp8_gemm(dyq, sdy, weight_t[0], weight_t[1], out_dtype=dx_dtype)
    dyt, sdyt = act_quant_t(dy)
    xt, sxt = act_quant_t(x)
    dw = fp8_gemm_rowwise(dyt, sdyt, xt, sxt, out_dtype=dw_dtype)
    return dx, dw
