"""GPU parity of the bf16 GEMM (the bf16 branch of linear(): the FP8 weight dequantised by
weight_dequant, then a plain bf16 linear) against the oracle's float64 bf16 linear, through
the C ABI. Tolerance (tests/helpers.py, bf16_linear_rel): every product is exact in fp32 and
the matrix unit sums them in fp32 32 at a time, so |y - y_hat| <= (K/32 + 1) 2^-24 sum |x w|
for fp32 output; bf16 output within 1 ulp of RN(y_hat), or within that bound plus one ulp
near cancellation."""
import numpy as np
import pytest
import torch

import fp8_act_quant_amd as fq
import oracle
import synth
from helpers import bf16_linear_rel, check_bf16_linear_every_output, dev_bf16, gemm_check, host_bits16, host_codes

pytestmark = pytest.mark.gpu

TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (37, 200, 384), (300, 576, 256), (256, 128, 64), (513, 129, 1024),
                                   (260, 1000, 1536), (130, 260, 448)])
def test_bf16_gemm_small_every_output(M, N, K, out, with_bias):
    X = synth.random_bf16((M, K), seed=M + 3 * N + K)
    W = synth.random_bf16((N, K), seed=5 * M + N + K, std=0.02)
    bias = np.random.Generator(np.random.PCG64(N + 1)).standard_normal(N).astype(np.float32) if with_bias else None
    y = fq.bf16_gemm(dev_bf16(X), dev_bf16(W), None if bias is None else torch.from_numpy(bias).cuda(),
                     out_dtype=TORCH_OUT[out])
    torch.cuda.synchronize()
    res = check_bf16_linear_every_output(y, X, W, out, f"bf16 gemm {M}x{N}x{K} {out} bias={with_bias}", bias)
    assert res["n"] == M * N
    # (with a bias, the one fp32 rounding of the addition is part of the bound: violations)
    assert res["violations"] == 0 and (with_bias or res["strict_violations"] == 0), res


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("K", [64, 320, 512])
def test_bf16_gemm_large_tile_every_output(K, out):
    """A shape with at least 256 tiles of 256x256 (17 x 17 here, ragged in both M and N),
    which takes the 8-wave 256x256 tile (A fragments streamed through each K step) rather
    than the 128x128 one; K of 1, 5 and 8 steps of 64."""
    M, N = 4100, 4097
    X = synth.random_bf16((M, K), seed=K + 11)
    W = synth.random_bf16((N, K), seed=K + 12, std=0.02)
    print(f"bf16 gemm large tile {M}x{N}x{K} {out}", flush=True)
    y = fq.bf16_gemm(dev_bf16(X), dev_bf16(W), out_dtype=TORCH_OUT[out])
    torch.cuda.synchronize()
    res = check_bf16_linear_every_output(y, X, W, out, f"bf16 gemm {M}x{N}x{K} {out}")
    assert res["n"] == M * N
    assert res["violations"] == 0 and res["strict_violations"] == 0, res


@pytest.mark.parametrize("tile", ["256x256", "128x128", "64x128"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (300, 260, 448), (513, 129, 1024), (257, 511, 128)])
def test_bf16_gemm_each_tile_every_output(tile, M, N, K, monkeypatch):
    """Each tile forced (FP8Q_BF16_TILE) on small ragged shapes, both output dtypes, with a
    bias: partial tiles in M and N, odd and even step counts."""
    monkeypatch.setenv("FP8Q_BF16_TILE", tile)
    X = synth.random_bf16((M, K), seed=7 * M + N + K)
    W = synth.random_bf16((N, K), seed=M + 5 * N + K, std=0.02)
    bias = np.random.Generator(np.random.PCG64(N + 9)).standard_normal(N).astype(np.float32)
    for out in ("f32", "bf16"):
        y = fq.bf16_gemm(dev_bf16(X), dev_bf16(W), torch.from_numpy(bias).cuda(), out_dtype=TORCH_OUT[out])
        torch.cuda.synchronize()
        res = check_bf16_linear_every_output(y, X, W, out, f"bf16 gemm {tile} {M}x{N}x{K} {out}", bias)
        assert res["n"] == M * N
        assert res["violations"] == 0, res


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_bf16_gemm_output_4_byte_aligned(out):
    """The interface asks only 4-byte alignment of y: an output 4 bytes past a 16-byte
    boundary (so no row of it is 16-byte aligned), through the C ABI, on every output."""
    from fp8_act_quant_amd import _lib as L
    M, N, K = 300, 264, 192
    X = synth.random_bf16((M, K), seed=41)
    W = synth.random_bf16((N, K), seed=42, std=0.02)
    x, w = dev_bf16(X), dev_bf16(W)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    per = 1 if out == "f32" else 2                    # elements in 4 bytes
    buf = torch.zeros(M * N + 8 * per, dtype=dt, device="cuda")
    assert buf.data_ptr() % 16 == 0
    y = buf[per:per + M * N].view(M, N)
    assert y.data_ptr() % 16 == 4
    code = L.FP8Q_OUT_F32 if out == "f32" else L.FP8Q_OUT_BF16
    for tile in ("256x256", "128x128", "64x128"):
        import os
        os.environ["FP8Q_BF16_TILE"] = tile
        try:
            assert fq.lib.fp8_bf16_gemm(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), code, M, N, K, None) == 0
            torch.cuda.synchronize()
        finally:
            del os.environ["FP8Q_BF16_TILE"]
        res = check_bf16_linear_every_output(y, X, W, out, f"bf16 gemm 4-byte aligned y {tile} {out}")
        assert res["violations"] == 0 and res["strict_violations"] == 0, (tile, res)
        assert torch.count_nonzero(buf[:per]) == 0 and torch.count_nonzero(buf[per + M * N:]) == 0


def test_bf16_gemm_k_zero_is_bias_and_empty_m():
    x = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((7, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.arange(7, dtype=torch.float32, device="cuda")
    y = fq.bf16_gemm(x, w, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, b.expand(5, 7))
    assert fq.bf16_gemm(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                        torch.zeros((3, 64), dtype=torch.bfloat16, device="cuda")).shape == (0, 3)


@pytest.mark.parametrize("name", ["q_down", "kv_down"])
def test_linear_bf16_branch_full_size_every_output(name):
    """linear(gemm_impl="bf16") at the projection's full size: the weight quantised and
    dequantised by the library (bit-exact with the oracle's weight_dequant), then every output
    of the bf16 GEMM (bf16 output, with a bias) against the oracle's bf16 linear."""
    wl = synth.WORKLOADS[name]
    X, W = synth.make_inputs(wl)
    print(f"linear bf16 branch {name} M={wl.M} N={wl.N} K={wl.K}", flush=True)
    bias = np.random.Generator(np.random.PCG64(3)).standard_normal(wl.N).astype(np.float32)
    x = dev_bf16(X)
    wq, sw = fq.weight_quant(dev_bf16(W))
    y = fq.linear(x, wq, torch.from_numpy(bias).cuda(), weight_scale=sw, gemm_impl="bf16")
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16 and y.shape == (wl.M, wl.N)
    wd = oracle.weight_dequant(host_codes(wq), sw.cpu().numpy())
    assert np.array_equal(host_bits16(fq.weight_dequant(wq, sw)), wd)
    res = check_bf16_linear_every_output(y, X, wd, "bf16", f"linear bf16 {name}", bias)
    assert res["n"] == wl.M * wl.N
    assert res["violations"] == 0, res


def test_linear_dispatch():
    """linear(): an FP8 weight with gemm_impl "fp8" is act_quant + the block GEMM with the bias
    fused; with gemm_impl "bf16" it is weight_dequant + the bf16 GEMM; a bf16 weight goes to the
    bf16 GEMM as it is; other weight dtypes, and an FP8 weight without its scale, are rejected."""
    M, N, K = 37, 300, 512
    x = dev_bf16(synth.random_bf16((M, K), seed=41))
    Wb = dev_bf16(synth.random_bf16((N, K), seed=42, std=0.02))
    bias = dev_bf16(synth.random_bf16((N,), seed=43))
    wq, sw = fq.weight_quant(Wb)
    q, s = fq.act_quant(x, scale_layout="kmajor")
    ref_fp8 = fq.fp8_gemm(q, s, wq, sw, out_dtype=torch.bfloat16, bias=bias)
    assert torch.equal(fq.linear(x, wq, bias, weight_scale=sw).view(torch.int16), ref_fp8.view(torch.int16))
    ref_bf16 = fq.bf16_gemm(x, fq.weight_dequant(wq, sw), bias)
    assert torch.equal(fq.linear(x, wq, bias, weight_scale=sw, gemm_impl="bf16").view(torch.int16),
                       ref_bf16.view(torch.int16))
    assert torch.equal(fq.linear(x, Wb, bias).view(torch.int16), fq.bf16_gemm(x, Wb, bias).view(torch.int16))
    # the bf16 branch against the oracle on every output
    res = check_bf16_linear_every_output(fq.linear(x, Wb, bias), host_bits16(x), host_bits16(Wb), "bf16",
                                         "linear bf16 weight", oracle.bf16_to_f32_array(host_bits16(bias)))
    assert res["violations"] == 0, res
    with pytest.raises(TypeError):
        fq.linear(x, Wb.float(), bias)
    with pytest.raises(ValueError):
        fq.linear(x, wq, bias)   # FP8 weight without its scale
    with pytest.raises(ValueError):
        fq.linear(x, wq, bias, weight_scale=sw, gemm_impl="fp16")
    with pytest.raises(ValueError):
        fq.fp8_gemm(q, s, wq, sw, bias=bias[:-1])


def test_bf16_gemm_deterministic_and_error_paths():
    from fp8_act_quant_amd import _lib as L
    X = dev_bf16(synth.random_bf16((700, 1024), 51))
    W = dev_bf16(synth.random_bf16((300, 1024), 52, std=0.02))
    y1 = fq.bf16_gemm(X, W)
    y2 = fq.bf16_gemm(X, W)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    g = fq.lib.fp8_bf16_gemm
    p = X.data_ptr()
    y = torch.empty((4, 4), dtype=torch.float32, device="cuda")
    assert g(p, p, None, y.data_ptr(), L.FP8Q_OUT_F32, 4, 4, 96, None) == L.FP8Q_ERR_SHAPE
    assert g(p, p, None, y.data_ptr(), 7, 4, 4, 64, None) == L.FP8Q_ERR_DTYPE
    assert g(p + 2, p, None, y.data_ptr(), L.FP8Q_OUT_F32, 4, 4, 64, None) == L.FP8Q_ERR_ALIGN
    assert g(None, p, None, y.data_ptr(), L.FP8Q_OUT_F32, 4, 4, 64, None) == L.FP8Q_ERR_NULL
    assert g(p, p, None, y.data_ptr(), L.FP8Q_OUT_F32, 4, 4, 1 << 23, None) == L.FP8Q_ERR_SHAPE
    with pytest.raises(ValueError):
        fq.bf16_gemm(X[:, :100].contiguous(), W[:, :100].contiguous())
    assert bf16_linear_rel(7168) == (224 + 1) * 2.0 ** -24


def test_bf16_gemm_maximum_k(monkeypatch):
    """The largest K the bf16 GEMM takes (2^23 - 64), on the 256x256 tile (forced): a
    256-row tile's byte offsets into X reach 255 * 2K + 2K - 16, just below 2^32. Sampled
    outputs, including the tile's last row and the ragged last column, against the oracle's
    float64 bf16 linear."""
    monkeypatch.setenv("FP8Q_BF16_TILE", "256x256")
    M, N, K = 256, 200, (1 << 23) - 64
    print(f"bf16 gemm maximum K {M}x{N}x{K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(21)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
    w = torch.randn((N, K), generator=g, device="cuda", dtype=torch.bfloat16) * 0.02
    for out in ("f32", "bf16"):
        y = fq.bf16_gemm(x, w, out_dtype=TORCH_OUT[out])
        torch.cuda.synchronize()
        rng = np.random.Generator(np.random.PCG64(22))
        rows = np.concatenate([[0, 127, 128, 255, 255, 255], rng.integers(0, M, 10)]).astype(np.int64)
        cols = np.concatenate([[0, 199, 128, 0, 127, 199], rng.integers(0, N, 10)]).astype(np.int64)
        uniq_r, uniq_c = np.unique(rows), np.unique(cols)
        xs = host_bits16(x[torch.from_numpy(uniq_r).cuda()])
        ws = host_bits16(w[torch.from_numpy(uniq_c).cuda()])
        y_hat, bound = oracle.matmul_bf16(xs, ws)
        ri = np.searchsorted(uniq_r, rows)
        ci = np.searchsorted(uniq_c, cols)
        yh = (y.float().cpu().numpy() if out == "f32" else host_bits16(y))[rows, cols]
        res = gemm_check(yh, y_hat[ri, ci], bound[ri, ci], out, rel=bf16_linear_rel(K))
        print(f"bf16 maximum K {out}", res, flush=True)
        assert res["violations"] == 0 and res["strict_violations"] == 0, (out, res)
