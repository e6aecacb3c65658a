"""GPU parity of fp8_act_quant_gemm (act_quant fused into the block GEMM) through the C ABI.

The fused call must produce the bytes of its two-call form: aq and sa bit-identical to
fp8_act_quant's, y bit-identical to fp8_block_gemm's on those codes (same tile plan), and
the GEMM within the stated bound of the CPU oracle. Shapes cover the fused path (the
q down-projection at full size, ragged M, short K below and around the quantisation lead)
and shapes that take the two-kernel path. Repeated calls on one workspace check that the
counters are left at zero, and the error word stays clear.
"""
import ctypes

import numpy as np
import pytest
import torch

import fp8_act_quant_amd as fq
import oracle
import synth
from fp8_act_quant_amd import _lib as L
from helpers import dev_bf16, gemm_check, host_bits16, host_codes, mfma_group_allowance, scale_floor

pytestmark = pytest.mark.gpu

ERROR_WORD = 4095


def _workspace(M, N, K, code):
    n = int(L.lib.fp8_act_quant_gemm_workspace_bytes(M, N, K, code))
    assert n >= 16384
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def _fused_call(x, wq, sw, out_dtype, ws, mode=0):
    M, K = x.shape
    N = wq.shape[0]
    code = (L.FP8Q_OUT_BF16 if out_dtype == torch.bfloat16 else L.FP8Q_OUT_F32) | mode
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=out_dtype, device="cuda")
    fused = ctypes.c_int(-1)
    rc = L.lib.fp8_act_quant_gemm(x.data_ptr(), aq.data_ptr(), sa.data_ptr(), wq.data_ptr(), sw.data_ptr(),
                                  y.data_ptr(), code, M, N, K, ws.data_ptr() if ws is not None else None,
                                  ws.numel() if ws is not None else 0, ctypes.byref(fused),
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == L.FP8Q_OK, L.lib.fp8q_strerror(rc)
    torch.cuda.synchronize()
    return y, aq, sa, fused.value


def _two_call(x, wq, sw, out_dtype, mode="default", workspace=None):
    """The two-call form. The fused kernel uses the plan without split-K; the two-kernel
    fallback uses the workspace it is given (split-K where the planner wants it), so compare
    that path with a workspace too (the fp32 summation order follows the split)."""
    aq, sa = fq.act_quant(x)
    y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=out_dtype, mode=mode, workspace=workspace)
    torch.cuda.synchronize()
    return y, aq, sa


def _same_bytes(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _weights(N, K, seed):
    W = synth.random_bf16((N, K), seed=seed, std=0.02)
    return fq.weight_quant(dev_bf16(W))


@pytest.mark.parametrize("M,N,K,expect_fused", [
    (4096, 1536, 7168, True),    # the q down-projection: 32 x 8 tiles of 128x192
    (4000, 1536, 7168, True),    # ragged last row band
    (4096, 1536, 640, True),     # 5 slices: all quantised in the prologue
    (4096, 1536, 768, True),     # 6 slices: one quantised in the loop
    (4096, 1536, 1408, True),    # 11 slices: loop and remainder
    (8192, 768, 1024, True),     # 4 tiles per row band (32 rows per workgroup)
    (4096, 576, 7168, False),    # 3 tiles per row band: two-kernel path
    (2048, 1536, 640, False),    # the planner's tile is 128x128: two-kernel path
    (300, 200, 512, False),      # a different tile: two-kernel path
])
def test_fused_matches_two_calls(M, N, K, expect_fused):
    x = dev_bf16(synth.random_bf16((M, K), seed=M + 7 * K))
    wq, sw = _weights(N, K, seed=N + 11 * K)
    ws = _workspace(M, N, K, L.FP8Q_OUT_BF16)
    y, aq, sa, fused = _fused_call(x, wq, sw, torch.bfloat16, ws)
    print(f"M={M} N={N} K={K} fused={fused}", flush=True)
    assert fused == int(expect_fused)
    y2, aq2, sa2 = _two_call(x, wq, sw, torch.bfloat16, workspace=None if fused else "auto")
    assert _same_bytes(aq, aq2), "codes differ from act_quant"
    assert _same_bytes(sa, sa2), "scales differ from act_quant"
    assert _same_bytes(y, y2), "output differs from the two-call GEMM"
    assert int(ws[ERROR_WORD * 4:ERROR_WORD * 4 + 4].view(torch.int32).item()) == 0
    assert int(ws[:16384].count_nonzero().item()) == 0, "counters not left at zero"


def test_fused_against_oracle_and_repeated_calls():
    """Three calls in a row on one workspace with different activations (the counters must
    be back at zero after each); the last output checked against the oracle on every
    element (bf16 output: within 1 bf16 ulp of the oracle plus the matrix-unit allowance)."""
    M, N, K = 4096, 1536, 1024
    wq, sw = _weights(N, K, seed=5)
    ws = _workspace(M, N, K, L.FP8Q_OUT_BF16)
    for seed in (1, 2, 3):
        A = synth.random_bf16((M, K), seed=seed)
        x = dev_bf16(A)
        y, aq, sa, fused = _fused_call(x, wq, sw, torch.bfloat16, ws)
        assert fused == 1
        y2, aq2, sa2 = _two_call(x, wq, sw, torch.bfloat16)
        assert _same_bytes(aq, aq2) and _same_bytes(sa, sa2) and _same_bytes(y, y2), seed
    # every element of the first and the last row band
    sel = np.r_[0:128, M - 128:M]
    haq, hsa, hwq, hsw = host_codes(aq)[sel], sa.cpu().numpy()[sel], host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.block_gemm(haq, hsa, hwq, hsw)
    R = len(sel)
    rows, cols = np.repeat(np.arange(R), N), np.tile(np.arange(N), R)
    allow = (scale_floor(haq, hwq, rows, cols) + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols)).reshape(R, N)
    res = gemm_check(host_bits16(y)[sel], y_hat, bound, "bf16", allow)
    assert res["violations"] == 0, res
    assert int(ws[:16384].count_nonzero().item()) == 0


def test_fused_fp32_output_fp8_products_and_exact_fallback():
    """fp32 output: with FP8 products forced the fused path runs; the default (exact
    slices) takes the two-kernel path. Both match their two-call forms bit for bit."""
    M, N, K = 4096, 1536, 1024
    x = dev_bf16(synth.random_bf16((M, K), seed=21))
    wq, sw = _weights(N, K, seed=22)
    ws = _workspace(M, N, K, L.FP8Q_OUT_F32 | L.FP8Q_GEMM_FP8_PRODUCTS)
    y, aq, sa, fused = _fused_call(x, wq, sw, torch.float32, ws, L.FP8Q_GEMM_FP8_PRODUCTS)
    assert fused == 1
    y2, _, _ = _two_call(x, wq, sw, torch.float32, mode="fp8")
    assert _same_bytes(y, y2)
    y, aq, sa, fused = _fused_call(x, wq, sw, torch.float32, ws)
    assert fused == 0
    y2, _, _ = _two_call(x, wq, sw, torch.float32, workspace="auto")
    assert _same_bytes(y, y2)


def test_fused_without_workspace_runs_two_kernels():
    M, N, K = 4096, 1536, 1024
    x = dev_bf16(synth.random_bf16((M, K), seed=31))
    wq, sw = _weights(N, K, seed=32)
    y, aq, sa, fused = _fused_call(x, wq, sw, torch.bfloat16, None)
    assert fused == 0
    y2, aq2, sa2 = _two_call(x, wq, sw, torch.bfloat16)
    assert _same_bytes(y, y2) and _same_bytes(aq, aq2) and _same_bytes(sa, sa2)


def test_fused_special_values_bit_exact():
    """Zero tiles, signed zeros, tiny and huge values and NaN in the activations: the fused
    quantiser's codes and scales equal act_quant's."""
    M, N, K = 4096, 1536, 1024
    A = synth.random_bf16((M, K), seed=41)
    bits = A.view(np.uint16).copy()
    bits[3, :128] = 0x0000                 # an all-zero tile
    bits[5, 128:256] = 0x8000              # all negative zeros
    bits[7, 256:384] = 0x0001              # subnormal bf16
    bits[9, 384] = 0x7F7F                  # the largest finite bf16
    bits[11, 512] = 0x7FC0                 # NaN
    bits[13, 640:768] = 0xC2C8             # constant tile
    x = dev_bf16(bits.view(A.dtype))
    wq, sw = _weights(N, K, seed=42)
    ws = _workspace(M, N, K, L.FP8Q_OUT_BF16)
    y, aq, sa, fused = _fused_call(x, wq, sw, torch.bfloat16, ws)
    assert fused == 1
    aq2, sa2 = fq.act_quant(x)
    torch.cuda.synchronize()
    assert _same_bytes(aq, aq2) and _same_bytes(sa, sa2)


def test_python_binding_act_quant_gemm():
    M, N, K = 4096, 1536, 1024
    x = dev_bf16(synth.random_bf16((M, K), seed=51))
    wq, sw = _weights(N, K, seed=52)
    y, q, s, fused = fq.act_quant_gemm(x, wq, sw, return_path=True)
    torch.cuda.synchronize()
    assert fused
    y2, q2, s2 = _two_call(x, wq, sw, torch.bfloat16)
    assert _same_bytes(y, y2) and _same_bytes(q, q2) and _same_bytes(s, s2)
