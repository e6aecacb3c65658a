"""GPU parity of the quantisation kernels against the CPU oracle, through the C ABI.

Codes and scales must be bit-identical: small shapes spanning several waves and a
ragged tail, hand-picked and golden tiles, every workload's full-size operands, and an
exhaustive sweep of all bf16 (x, amax) pairs through the real act_quant kernel.
"""
import json
import os
import time

import numpy as np
import pytest
import torch

import fp8_act_quant_amd as fq
import oracle
import synth
from helpers import dev_bf16, dev_codes, dev_f32, host_bits16, host_codes, host_f32_bits

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_act_quant(A):
    q, s = fq.act_quant(dev_bf16(A))
    torch.cuda.synchronize()
    return host_codes(q), host_f32_bits(s)


def gpu_weight_quant(W):
    q, s = fq.weight_quant(dev_bf16(W))
    torch.cuda.synchronize()
    return host_codes(q), host_f32_bits(s)


def assert_act_parity(A, label=""):
    q, s = gpu_act_quant(A)
    oq, os_ = oracle.act_quant(A)
    bad_q = np.count_nonzero(q != oq)
    bad_s = np.count_nonzero(s != os_.view(np.uint32))
    assert bad_q == 0 and bad_s == 0, f"{label}: {bad_q} codes and {bad_s} scales differ"


def assert_weight_parity(W, label=""):
    q, s = gpu_weight_quant(W)
    oq, os_ = oracle.weight_quant(W)
    bad_q = np.count_nonzero(q != oq)
    bad_s = np.count_nonzero(s != os_.view(np.uint32))
    assert bad_q == 0 and bad_s == 0, f"{label}: {bad_q} codes and {bad_s} scales differ"


# ------------------------------------------------------------------------------ act_quant

@pytest.mark.parametrize("M,K", [(1, 128), (3, 128), (37, 384), (64, 256), (257, 1024), (1000, 7168)])
def test_act_quant_small_shapes(M, K):
    assert_act_parity(synth.random_bf16((M, K), seed=M * 7 + K), f"{M}x{K}")


def test_act_quant_wide_dynamic_range():
    rng = np.random.Generator(np.random.PCG64(5))
    a = rng.standard_normal((96, 1024)).astype(np.float32)
    a *= np.exp2(rng.integers(-140, 120, size=(96, 8, 1)).astype(np.float32)).repeat(128, axis=2).reshape(96, 1024)
    assert_act_parity(synth.bf16_bits(a), "per-tile exponents 2^-140..2^120")


def test_act_quant_special_tiles():
    assert_act_parity(synth.special_tiles(), "special tiles")


def test_act_quant_golden_tiles():
    cases = json.load(open(os.path.join(GOLDEN, "act_quant_cases.json")))["cases"]
    x = np.zeros((len(cases), 128), dtype=np.uint16)
    for i, c in enumerate(cases):
        for j, h in c["tile"]:
            x[i, j] = int(h, 16)
    q, s = gpu_act_quant(x)
    for i, c in enumerate(cases):
        assert int(s[i, 0]) == int(c["scale_bits"], 16), c["name"]
        for j, code in c["codes"]:
            assert q[i, j] == int(code, 16), (c["name"], j)


def test_act_quant_empty():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = fq.act_quant(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


def test_act_quant_leading_dims_flattened():
    A = synth.random_bf16((2, 3, 512), seed=3)
    q, s = fq.act_quant(dev_bf16(A))
    torch.cuda.synchronize()
    oq, os_ = oracle.act_quant(A.reshape(6, 512))
    assert q.shape == (2, 3, 512) and s.shape == (2, 3, 4)
    assert np.array_equal(host_codes(q).reshape(6, 512), oq)
    assert np.array_equal(host_f32_bits(s).reshape(6, 4), os_.view(np.uint32))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_act_quant_workload_full_size(name):
    A, _ = synth.make_inputs(name, with_weight=False)
    print(f"act_quant parity {name} {A.shape}", flush=True)
    assert_act_parity(A, name)


# nkb = K/128 from 1 to 129 (powers of two and their neighbours, odd counts), ragged M
@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (37, 384), (5, 640), (257, 7168), (1000, 128 * 57),
                                 (64, 128 * 63), (33, 128 * 64), (17, 128 * 65), (9, 128 * 129)])
def test_act_quant_kmajor_small_shapes(M, K):
    """fp8_act_quant_kmajor: the oracle's codes, and its scale grid transposed, bit for bit."""
    A = synth.random_bf16((M, K), seed=M * 13 + K)
    q, s = fq.act_quant(dev_bf16(A), scale_layout="kmajor")
    torch.cuda.synchronize()
    assert s.shape == (M, K // 128) and s.movedim(-1, 0).is_contiguous()
    oq, os_ = oracle.act_quant(A)
    assert np.array_equal(host_codes(q), oq), f"{M}x{K}: codes differ"
    st = host_f32_bits(s.movedim(-1, 0))
    assert np.array_equal(st, np.ascontiguousarray(os_.T).view(np.uint32)), f"{M}x{K}: scales differ"


def test_act_quant_kmajor_leading_dims_and_empty():
    A = synth.random_bf16((2, 3, 512), seed=4)
    q, s = fq.act_quant(dev_bf16(A), scale_layout="kmajor")
    torch.cuda.synchronize()
    oq, os_ = oracle.act_quant(A.reshape(6, 512))
    assert q.shape == (2, 3, 512) and s.shape == (2, 3, 4)
    assert np.array_equal(host_codes(q).reshape(6, 512), oq)
    assert np.array_equal(host_f32_bits(s.contiguous()).reshape(6, 4), os_.view(np.uint32))
    q, s = fq.act_quant(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"), scale_layout="kmajor")
    assert q.shape == (0, 256) and s.shape == (0, 2)
    with pytest.raises(ValueError):
        fq.act_quant(dev_bf16(A), scale_layout="col")


def test_act_quant_kmajor_workload_full_size():
    """The benchmark's act_quant (query down-projection activations) in the K-block-major
    layout it runs with, against the oracle."""
    A, _ = synth.make_inputs("q_down", with_weight=False)
    q, s = fq.act_quant(dev_bf16(A), scale_layout="kmajor")
    torch.cuda.synchronize()
    oq, os_ = oracle.act_quant(A)
    assert np.array_equal(host_codes(q), oq)
    assert np.array_equal(host_f32_bits(s.movedim(-1, 0)), np.ascontiguousarray(os_.T).view(np.uint32))


def test_act_quant_kmajor_large_tile_index():
    """About 2^24 tiles (K/128 = 57): the tile -> (row, K slice) division at large tile
    numbers, against the row-major kernel on the same input (bit-exact against the oracle
    above): equal codes, and scales that are the transpose of each other."""
    M, K = 300007, 128 * 57
    print(f"act_quant kmajor vs row-major {M}x{K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    qr, sr = fq.act_quant(x)
    qk, sk = fq.act_quant(x, scale_layout="kmajor")
    torch.cuda.synchronize()
    assert torch.equal(qr.view(torch.uint8), qk.view(torch.uint8))
    assert torch.equal(sr.view(torch.int32), sk.contiguous().view(torch.int32))
    del x, qr, qk


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_act_quant_exhaustive_bf16_pairs():
    """Every bf16 (x, amax) pair with |x| <= amax, both signs, through the kernel."""
    t0 = time.time()
    total = 0
    for lo, hi in synth.exhaustive_chunks(max_tiles=1 << 19):
        tiles = synth.exhaustive_tiles(lo, hi)
        q, s = gpu_act_quant(tiles)
        oq, os_ = oracle.act_quant(tiles)
        bad = np.nonzero((q != oq).any(axis=1) | (s[:, 0] != os_[:, 0].view(np.uint32)))[0]
        assert bad.size == 0, (f"amax patterns [{lo:#x}, {hi:#x}): {bad.size} tiles differ, first tile "
                               f"{tiles[bad[0], :4]} codes {q[bad[0], :4]} vs {oq[bad[0], :4]}")
        total += tiles.shape[0]
    print(f"exhaustive: {total} tiles ({total * 127} pairs) bit-exact in {time.time() - t0:.1f}s", flush=True)
    assert total == synth.exhaustive_tile_count(1, synth.EXHAUSTIVE_AB_MAX + 1)


# ------------------------------------------------------------------------------ weight_quant

@pytest.mark.parametrize("N,K", [(1, 128), (64, 128), (130, 256), (200, 384), (576, 7168), (1536, 512)])
def test_weight_quant_small_shapes(N, K):
    assert_weight_parity(synth.random_bf16((N, K), seed=N + 3 * K, std=0.02), f"{N}x{K}")


def test_weight_quant_wide_dynamic_range():
    rng = np.random.Generator(np.random.PCG64(6))
    w = rng.standard_normal((384, 512)).astype(np.float32)
    e = rng.integers(-140, 120, size=(3, 1, 4, 1)).astype(np.float32)
    w = (w.reshape(3, 128, 4, 128) * np.exp2(e)).reshape(384, 512)
    assert_weight_parity(synth.bf16_bits(w), "per-block exponents")


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_weight_quant_workload_full_size(name):
    _, W = synth.make_inputs(name)
    print(f"weight_quant parity {name} {W.shape}", flush=True)
    assert_weight_parity(W, name)


# ------------------------------------------------------------------------------ dequant

def gpu_dequant(q, s):
    w = fq.weight_dequant(dev_codes(q), dev_f32(s))
    torch.cuda.synchronize()
    return host_bits16(w)


def test_dequant_all_codes_all_scale_ranges():
    # every finite code against scales spanning the fp32 range (products that are fp32
    # subnormal, round to bf16 subnormals, or approach the bf16 maximum)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    N, K = 130, 256 * 4
    q = np.resize(codes, (N, K))
    rng = np.random.Generator(np.random.PCG64(8))
    s = (rng.uniform(1, 2, size=(2, 8)) * np.exp2(rng.integers(-149, 119, size=(2, 8)))).astype(np.float32)
    s[0, 0] = 1.0
    s[1, 1] = 0.0
    s[0, 2] = np.float32(2.0 ** -149)
    s[0, 3] = np.float32(3.389e38 / 448)
    assert np.array_equal(gpu_dequant(q, s), oracle.weight_dequant(q, s))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_dequant_workload_full_size(name):
    _, W = synth.make_inputs(name)
    q, s = oracle.weight_quant(W)
    assert np.array_equal(gpu_dequant(q, s), oracle.weight_dequant(q, s))


def test_weight_quant_and_dequant_maximum_block_rows():
    """65535 block rows, the most weight_quant's grid takes (N = 128 * 65535 - 64: a ragged
    last block row), K = 256. Sampled block rows (the first, the last, and others) against the
    oracle on those rows (blocks are independent), codes, scales and the dequantised weight,
    bit for bit; the dequant runs its grid-stride loop many times at this size."""
    N, K = 128 * 65535 - 64, 256
    print(f"weight_quant / dequant {N}x{K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(21)
    w = (0.02 * torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
    q, sc = fq.weight_quant(w)
    wd = fq.weight_dequant(q, sc)
    torch.cuda.synchronize()
    nnb = (N + 127) // 128
    assert sc.shape == (nnb, K // 128)
    rng = np.random.Generator(np.random.PCG64(22))
    for nb in [0, 1, nnb // 2, nnb - 2, nnb - 1] + list(rng.integers(0, nnb, 8)):
        r0, r1 = 128 * int(nb), min(128 * int(nb) + 128, N)
        wb = host_bits16(w[r0:r1])
        oq, os_ = oracle.weight_quant(wb)
        assert np.array_equal(host_codes(q[r0:r1]), oq), nb
        assert np.array_equal(host_f32_bits(sc[nb:nb + 1]), os_.view(np.uint32)), nb
        assert np.array_equal(host_bits16(wd[r0:r1]), oracle.weight_dequant(oq, os_)), nb
    del w, q, wd


def test_quant_error_paths_on_device():
    x = torch.zeros(4, 256 + 8, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(4 * 256 + 16, dtype=torch.uint8, device="cuda")
    s = torch.empty(16, dtype=torch.float32, device="cuda")
    from fp8_act_quant_amd import _lib as L
    assert fq.lib.fp8_act_quant(x.data_ptr() + 2, q.data_ptr(), s.data_ptr(), 4, 256, None) == L.FP8Q_ERR_ALIGN
    assert fq.lib.fp8_act_quant(x.data_ptr(), q.data_ptr() + 1, s.data_ptr(), 4, 256, None) == L.FP8Q_ERR_ALIGN
    assert fq.lib.fp8_act_quant(x.data_ptr(), q.data_ptr(), s.data_ptr(), 4, 200, None) == L.FP8Q_ERR_SHAPE
    with pytest.raises(fq.Fp8qError):
        L.check("fp8_act_quant", fq.lib.fp8_act_quant(x.data_ptr(), q.data_ptr(), 0, 4, 256, None))
