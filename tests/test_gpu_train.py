"""GPU parity of the FP8 training-side kernels against the CPU oracle, through the C ABI:
token-wise quantisation with a transposed output (bit-exact), the FP8 weight transpose
(bit-exact), the GEMM with per-row scales on both operands (the stated GEMM tolerance, both
contraction modes), and linear()'s backward at the q down-projection's full size (sampled).
"""
import numpy as np
import pytest
import torch

import fp8_act_quant_amd as fq
import oracle
import synth
from helpers import (check_every_output, dev_bf16, gemm_check, group_allowance_applies, host_bits16, host_codes,
                     mfma_group_allowance_rowwise, scale_floor)

pytestmark = pytest.mark.gpu

TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16}


def y_host(y, out):
    return y.float().cpu().numpy() if out == "f32" else host_bits16(y)


def special_bf16(M, C, seed):
    """Random bf16 with per-channel magnitudes spread over 2^-30 .. 2^20, some zero channels
    and a few tokens at exact powers of two (ties and saturation boundaries)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, C)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 20, size=(1, C))).astype(np.float32)
    x[:, ::7] = 0.0
    x[::13, 1::5] = np.float32(448.0)
    return synth.bf16_bits(x)


@pytest.mark.parametrize("M,C", [(1, 8), (130, 64), (300, 136), (128, 1024), (4097, 520)])
def test_act_quant_t_bit_exact(M, C):
    x = special_bf16(M, C, seed=M + C)
    qt, st = fq.act_quant_t(dev_bf16(x))
    torch.cuda.synchronize()
    oq, os_ = oracle.act_quant_t(x)
    assert qt.shape == oq.shape and st.shape == os_.shape
    gq = host_codes(qt)
    assert np.array_equal(gq, oq), int((gq != oq).sum())
    assert np.array_equal(st.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("N,K", [(1, 128), (256, 384), (576, 1024), (100, 256), (1536, 7168)])
def test_weight_transpose_bit_exact(N, K):
    w = synth.random_bf16((N, K), seed=N + K, std=0.02)
    wq, sw = fq.weight_quant(dev_bf16(w))
    wqt, swt = fq.weight_transpose(wq, sw)
    torch.cuda.synchronize()
    oq, os_ = oracle.weight_transpose(host_codes(wq), sw.cpu().numpy())
    assert np.array_equal(host_codes(wqt), oq)
    assert np.array_equal(swt.cpu().numpy().view(np.uint32), os_.view(np.uint32))


def test_act_quant_t_and_weight_transpose_large():
    """act_quant_t over 2^22 + 3 tokens (32769 token blocks along the grid's x, a ragged
    last block) and weight_transpose at the most 64-row tiles its grid's y takes (N = 64 *
    65535 - 10). Sampled token blocks against the oracle on those tokens (blocks are
    independent), and sampled column ranges of the transposed weight and its scale grid."""
    g = torch.Generator(device="cuda").manual_seed(31)
    M, C = (1 << 22) + 3, 64
    print(f"act_quant_t {M}x{C}", flush=True)
    x = torch.randn((M, C), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    qt, st = fq.act_quant_t(x)
    torch.cuda.synchronize()
    nmb = (M + 127) // 128
    assert qt.shape == (C, nmb * 128) and st.shape == (C, nmb)
    rng = np.random.Generator(np.random.PCG64(32))
    for mb in [0, 1, nmb // 2, nmb - 1] + list(rng.integers(0, nmb, 6)):
        t0, t1 = 128 * int(mb), min(128 * int(mb) + 128, M)
        oq, os_ = oracle.act_quant_t(host_bits16(x[t0:t1]))
        assert np.array_equal(host_codes(qt[:, 128 * mb:128 * mb + 128].contiguous()), oq), mb
        assert np.array_equal(st[:, mb:mb + 1].contiguous().cpu().numpy().view(np.uint32), os_.view(np.uint32)), mb
    del x, qt, st
    N, K = 64 * 65535 - 10, 256
    print(f"weight_transpose {N}x{K}", flush=True)
    w = (0.02 * torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
    wq, sw = fq.weight_quant(w)
    del w
    wqt, swt = fq.weight_transpose(wq, sw)
    torch.cuda.synchronize()
    assert wqt.shape == (K, N) and swt.shape == (K // 128, (N + 127) // 128)
    for n0 in [0, 64, N // 2 - N // 2 % 64, N - 300] + [int(v) * 64 for v in rng.integers(0, N // 64, 4)]:
        n1 = min(n0 + 300, N)
        assert np.array_equal(host_codes(wqt[:, n0:n1].contiguous()), host_codes(wq[n0:n1]).T), n0
    assert torch.equal(swt.view(torch.int32), sw.t().contiguous().view(torch.int32))


class RowwiseReference:
    """The oracle's full per-row GEMM and the per-output allowances of one operand set
    (computed once, reused across modes and configurations)."""

    def __init__(self, aq, sa, bq, sb):
        haq, hsa, hbq, hsb = host_codes(aq), sa.cpu().numpy(), host_codes(bq), sb.cpu().numpy()
        self.y_hat, self.bound = oracle.rowwise_gemm(haq, hsa, hbq, hsb)
        M, N = self.y_hat.shape
        rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
        self.floor = scale_floor(haq, hbq, rows, cols).reshape(M, N)
        self.fp8 = self.floor + mfma_group_allowance_rowwise(haq, hsa, hbq, hsb, rows, cols).reshape(M, N)

    def check(self, y, out, mode):
        return gemm_check(y_host(y, out), self.y_hat, self.bound, out,
                          self.fp8 if group_allowance_applies(mode, out) else self.floor)


def rowwise_check(aq, sa, bq, sb, y, out, mode):
    return RowwiseReference(aq, sa, bq, sb).check(y, out, mode)


@pytest.mark.parametrize("mode", ["exact", "fp8"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (37, 200, 384), (300, 576, 1024), (1, 1, 2048)])
def test_rowwise_gemm_small_full_output(M, N, K, out, mode):
    A = synth.random_bf16((M, K), seed=3 * M + K)
    B = synth.random_bf16((N, K), seed=5 * N + K)
    aq, sa = fq.act_quant(dev_bf16(A))
    bq, sb = fq.act_quant(dev_bf16(B))   # per-row scales on the second operand
    y = fq.fp8_gemm_rowwise(aq, sa, bq, sb, out_dtype=TORCH_OUT[out], mode=mode)
    torch.cuda.synchronize()
    res = rowwise_check(aq, sa, bq, sb, y, out, mode)
    print(f"rowwise {M}x{N}x{K} {out} {mode}", res, flush=True)
    assert res["violations"] == 0, res


@pytest.mark.parametrize("M,N,K", [(300, 576, 2048), (129, 200, 1280)])
def test_rowwise_every_tile_configuration(M, N, K):
    """Every configuration the planner can choose for per-row scales, forced in turn, with
    and without split-K; configurations without a per-row instantiation fall back to the
    default one, which must be correct too."""
    from fp8_act_quant_amd import _lib as L
    A = synth.random_bf16((M, K), seed=M + 2 * K)
    B = synth.random_bf16((N, K), seed=N + 3 * K)
    aq, sa = fq.act_quant(dev_bf16(A))
    bq, sb = fq.act_quant(dev_bf16(B))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    ref = RowwiseReference(aq, sa, bq, sb)
    names = []
    while (n := fq.lib.fp8q_gemm_config_name(len(names))) is not None:
        names.append(n.decode())
    try:
        for c, name in enumerate(names):
            for splits in (1, 2):
                assert fq.lib.fp8q_gemm_force_config(c, splits) == L.FP8Q_OK
                for out, mode in (("bf16", "fp8"), ("f32", "exact")):
                    y = fq.fp8_gemm_rowwise(aq, sa, bq, sb, out_dtype=TORCH_OUT[out], mode=mode, workspace=ws)
                    torch.cuda.synchronize()
                    res = ref.check(y, out, mode)
                    print(f"rowwise config {name} splits {splits} {out} {mode}", res, flush=True)
                    assert res["violations"] == 0, (name, splits, out, mode, res)
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


def test_linear_backward_q_down_full_size_every_output():
    """Backward of the q down-projection (4096 tokens, 7168 -> 1536) at full size: the
    codes the kernels consumed are the oracle's, dX is checked against the block GEMM through
    the transposed weight and dW against the per-row GEMM over tokens, on every output."""
    wl = synth.WORKLOADS["q_down"]
    X, W = synth.make_inputs(wl)
    dY = synth.random_bf16((wl.M, wl.N), seed=101)
    print(f"linear backward q_down M={wl.M} N={wl.N} K={wl.K}", flush=True)
    x, dy = dev_bf16(X), dev_bf16(dY)
    wq, sw = fq.weight_quant(dev_bf16(W))
    dx, dw = fq.linear_backward(dy, x, wq, sw)
    torch.cuda.synchronize()
    assert dx.shape == (wl.M, wl.K) and dx.dtype == torch.bfloat16
    assert dw.shape == (wl.N, wl.K) and dw.dtype == torch.float32
    # dX = dY . W
    dyq, sdy = oracle.act_quant(dY)
    wqt, swt = oracle.weight_transpose(host_codes(wq), sw.cpu().numpy())
    res = check_every_output(dx, dyq, sdy, wqt, swt, "bf16", "dX")
    assert res["n"] == wl.M * wl.K
    assert res["violations"] == 0 and res["strict_violations"] == 0, res
    # dW = dY^T . X over tokens (fp32 output: exact slices)
    dyt, sdyt = oracle.act_quant_t(dY)
    xt, sxt = oracle.act_quant_t(X)
    gq, _ = fq.act_quant_t(x)
    assert np.array_equal(host_codes(gq), xt)
    res = check_every_output(dw, dyt, sdyt, xt, sxt, "f32", "dW", rowwise=True)
    assert res["n"] == wl.N * wl.K
    assert res["violations"] == 0 and res["strict_violations"] == 0, res
    assert torch.isfinite(dx.float()).all() and torch.isfinite(dw).all()


def test_training_error_paths():
    from fp8_act_quant_amd import _lib as L
    x = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((16, 128), dtype=torch.uint8, device="cuda")
    s = torch.empty((16, 1), dtype=torch.float32, device="cuda")
    assert fq.lib.fp8_act_quant_t(x.data_ptr(), q.data_ptr(), s.data_ptr(), 4, 12, None) == L.FP8Q_ERR_SHAPE
    assert fq.lib.fp8_act_quant_t(x.data_ptr() + 2, q.data_ptr(), s.data_ptr(), 4, 16, None) == L.FP8Q_ERR_ALIGN
    assert fq.lib.fp8_act_quant_t(None, q.data_ptr(), s.data_ptr(), 4, 16, None) == L.FP8Q_ERR_NULL
    assert fq.lib.fp8_act_quant_t(None, None, None, 0, 16, None) == L.FP8Q_OK
    assert fq.lib.fp8_weight_transpose(q.data_ptr(), s.data_ptr(), q.data_ptr(), s.data_ptr(), 16, 100, None) == \
        L.FP8Q_ERR_SHAPE
    y = torch.empty((4, 4), dtype=torch.float32, device="cuda")
    assert fq.lib.fp8_rowwise_gemm(q.data_ptr(), s.data_ptr(), q.data_ptr(), s.data_ptr(), y.data_ptr(), 7, 4, 4, 128,
                                   None, 0, None) == L.FP8Q_ERR_DTYPE
    assert fq.lib.fp8_rowwise_gemm(q.data_ptr(), s.data_ptr(), q.data_ptr(), s.data_ptr(), y.data_ptr(), 0, 4, 4, 100,
                                   None, 0, None) == L.FP8Q_ERR_SHAPE
    with pytest.raises(ValueError):
        fq.act_quant_t(torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda"))
