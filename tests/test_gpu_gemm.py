"""GPU parity of the block-scaled GEMM against the CPU oracle, through the C ABI.

The GPU and the oracle see the same codes and scales (produced by the GPU quantisers,
whose bit-exactness is checked separately). Small shapes are compared on every output in
both contraction modes, the workloads at full size on every output in the default mode
and launch configuration the benchmark uses. Tolerances: see tests/helpers.py (the stated
bound; plus, only where a test explicitly asks for FP8 products with fp32 output, the
measured matrix-unit allowance).
"""
import json
import os

import numpy as np
import pytest
import torch

import fp8_act_quant_amd as fq
import oracle
import synth
from helpers import (check_every_output, dev_bf16, dev_codes, dev_f32, gemm_check, group_allowance_applies,
                     host_bits16, host_codes, mfma_group_allowance, rel_error_vs_unquantised, scale_floor)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16}


def quantise_on_gpu(A, W):
    aq, sa = fq.act_quant(dev_bf16(A))
    wq, sw = fq.weight_quant(dev_bf16(W))
    return aq, sa, wq, sw


def y_host(y, out):
    return y.float().cpu().numpy() if out == "f32" else host_bits16(y)


def run_full_check(A, W, out, label, mode="default"):
    """Full-output check. Every result must meet the stated bound, except an explicit
    FP8-product request with fp32 output, which gets the matrix-unit allowance on top."""
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode)
    torch.cuda.synchronize()
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.block_gemm(haq, hsa, hwq, hsw)
    M, N = y_hat.shape
    rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    allowance = scale_floor(haq, hwq, rows, cols).reshape(M, N)
    if group_allowance_applies(mode, out):
        allowance = allowance + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols).reshape(M, N)
    res = gemm_check(y_host(y, out), y_hat, bound, out, allowance)
    print(label, mode, res, flush=True)
    assert res["violations"] == 0, (label, mode, res)
    return y


@pytest.mark.parametrize("mode", ["exact", "fp8"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (1, 1, 128), (37, 200, 384), (129, 129, 128),
                                   (300, 576, 256), (130, 64, 1024), (256, 384, 2048), (8, 1000, 128)])
def test_gemm_small_full_output(M, N, K, out, mode):
    A = synth.random_bf16((M, K), seed=M + N + K)
    W = synth.random_bf16((N, K), seed=M * N + K, std=0.02)
    run_full_check(A, W, out, f"{M}x{N}x{K} {out}", mode)


def test_gemm_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    A, W = synth.make_inputs(wl)
    run_full_check(A, W, wl.out_dtype, "tiny")


def test_gemm_golden_small():
    g = json.load(open(os.path.join(GOLDEN, "gemm_small.json")))
    K = g["K"]

    def rows(spec):
        out = np.zeros((len(spec["rows"]), K), dtype=np.uint16)
        for i, r in enumerate(spec["rows"]):
            out[i] = int(r["fill"], 16)
            for k, h in r["set"]:
                out[i, k] = int(h, 16)
        return out

    aq, sa, wq, sw = quantise_on_gpu(rows(g["A"]), rows(g["W"]))
    y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), np.array(g["Y"]))


def test_gemm_k_zero_writes_zeros():
    a = torch.empty((5, 0), dtype=torch.float8_e4m3fn, device="cuda")
    sa = torch.empty((5, 0), dtype=torch.float32, device="cuda")
    w = torch.empty((7, 0), dtype=torch.float8_e4m3fn, device="cuda")
    sw = torch.empty((1, 0), dtype=torch.float32, device="cuda")
    y = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda")
    fq.fp8_gemm(a, sa, w, sw, out_dtype=torch.float32, out=y)
    assert torch.all(y == 0)


def test_gemm_empty_m():
    a = torch.empty((0, 128), dtype=torch.float8_e4m3fn, device="cuda")
    sa = torch.empty((0, 1), dtype=torch.float32, device="cuda")
    w = torch.zeros((3, 128), dtype=torch.float8_e4m3fn, device="cuda")
    sw = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    assert fq.fp8_gemm(a, sa, w, sw).shape == (0, 3)


@pytest.mark.parametrize("mode", ["exact", "fp8"])
def test_gemm_one_hot_rows(mode):
    # one non-zero per A row: y[m, n] is a single E4M3 product times sa * sw, which
    # checks the scale indexing and the ragged N-block directly; the 0x0003 row (a bf16
    # subnormal) drives sa * sw below the fp32 normal range
    M, N, K = 6, 300, 512
    A = np.zeros((M, K), dtype=np.uint16)
    for m, (k0, v) in enumerate(zip([0, 127, 128, 300, 383, 511], [0x3F80, 0xC2F6, 0x0003, 0x7F7F, 0xBC00, 0x4123])):
        A[m, k0] = v
    W = synth.random_bf16((N, K), 8, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode=mode).cpu().numpy()
    haq, hwq = host_codes(aq), host_codes(wq)
    y_hat, bound = oracle.block_gemm(haq, sa.cpu().numpy(), hwq, sw.cpu().numpy())
    rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    floor = scale_floor(haq, hwq, rows, cols).reshape(M, N)
    res = gemm_check(y, y_hat, bound, "f32", floor)
    assert res["violations"] == 0, res
    normal = np.array([m != 2 for m in range(M)])
    assert np.all(np.abs(y - y_hat)[normal] <= 2.0 ** -23 * np.abs(y_hat)[normal])


def test_gemm_power_of_two_scales_exact():
    # E4M3 values times power-of-two scales: quantisation is lossless. Each A row and each
    # W block row keeps one exponent across K slices; the +-448 pins of A (k = 1) and W
    # (k = 0) sit alone in their group of 8 k (the rest of k = 0..7 is zero), so no group
    # mixes magnitudes beyond what the matrix unit adds exactly, every slice partial needs
    # <= 20 bits and the fp32 accumulation of the two slices is exact: Y == A . W^T.
    rng = np.random.Generator(np.random.PCG64(12))
    dec = oracle.e4m3_decode_all()
    small = np.array([c for c in range(256) if c not in (0x7F, 0xFF) and abs(dec[c]) <= 8
                      and (dec[c] * 8) % 1 == 0], dtype=np.uint8)
    M, N, K = 64, 260, 256
    ca = rng.choice(small, size=(M, K))
    cw = rng.choice(small, size=(N, K))
    for kb in range(K // 128):
        ca[:, 128 * kb:128 * kb + 8] = 0
        cw[:, 128 * kb:128 * kb + 8] = 0
    ca[:, 1::128] = 0x7E
    cw[::128, ::128] = 0xFE
    ea = np.repeat(rng.integers(-2, 3, size=(M, 1)), K // 128, axis=1)
    ew = np.repeat(rng.integers(-2, 3, size=((N + 127) // 128, 1)), K // 128, axis=1)
    a64 = dec[ca] * np.repeat(2.0 ** ea, 128, axis=1)
    w64 = dec[cw] * np.repeat(2.0 ** ew, 128, axis=1)[np.arange(N) // 128]
    aq, sa, wq, sw = quantise_on_gpu(synth.bf16_bits(a64.astype(np.float32)), synth.bf16_bits(w64.astype(np.float32)))
    assert np.array_equal(sa.cpu().numpy(), np.float32(2.0 ** ea))
    for mode in ("exact", "fp8"):
        y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode=mode).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, a64 @ w64.T), mode


def test_matrix_unit_group_alignment():
    # Documents the measured FP8 matrix-unit behaviour behind mfma_group_allowance: with
    # unit scales, a 2^-9 product in the same group of 8 k as a 448 product is dropped
    # (truncated to a multiple of 2^(8 - 13)), while in the next group it is kept. The
    # exact-slice mode returns every sum exactly.
    K = 128
    aq = np.zeros((4, K), dtype=np.uint8)
    aq[0, 0], aq[0, 1] = 0x7E, 0x01          # 448 and 2^-9, same group
    aq[1, 0], aq[1, 8] = 0x7E, 0x01          # different groups
    aq[2, 0], aq[2, 1] = 0x7E, 0x21          # 448 + 0.140625 -> 448.125 (multiple of 2^-5)
    aq[3, 0], aq[3, 1], aq[3, 2] = 0x7E, 0xFE, 0x01   # 448 - 448 + 2^-9 -> 0
    wq = np.full((1, K), 0x38, dtype=np.uint8)       # 1.0
    args = (dev_codes(aq), dev_f32(np.ones((4, 1))), dev_codes(wq), dev_f32(np.ones((1, 1))))
    fp8 = fq.fp8_gemm(*args, out_dtype=torch.float32, mode="fp8").cpu().numpy()[:, 0].astype(np.float64)
    exact = fq.fp8_gemm(*args, out_dtype=torch.float32, mode="exact").cpu().numpy()[:, 0].astype(np.float64)
    assert list(fp8) == [448.0, 448.0 + 2.0 ** -9, 448.125, 0.0], fp8
    assert list(exact) == [448.0 + 2.0 ** -9, 448.0 + 2.0 ** -9, 448.140625, 2.0 ** -9], exact


@pytest.mark.parametrize("mode", ["exact", "fp8"])
def test_gemm_deterministic(mode):
    A = synth.random_bf16((300, 1024), 21)
    W = synth.random_bf16((576, 1024), 22, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    y1 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode=mode)
    y2 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode=mode)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("M,N,K", [(300, 576, 2048), (513, 777, 3072), (1, 1, 2048), (129, 129, 1280)])
def test_gemm_split_k_workspace(M, N, K):
    """Shapes with few output tiles split K over several workgroups when a workspace is
    given. The split result meets the bound like the unsplit one, repeats bit for bit
    with a reused workspace (also after the workspace served another shape, and after its
    whole contents were overwritten with random bytes: the arrival words carry a per-launch
    epoch, so no contents count as arrivals), and differs from the unsplit result only by
    fp32 rounding order."""
    need = fq.gemm_workspace_bytes(M, N, K, torch.bfloat16)
    assert need > 0, "shape expected to use split-K"
    A = synth.random_bf16((M, K), seed=7 * M + K)
    W = synth.random_bf16((N, K), seed=11 * N + K, std=0.02)
    print(f"split-K {M}x{N}x{K} workspace {need} B", flush=True)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    gen = torch.Generator(device="cuda").manual_seed(M + N + K)
    ws = torch.randint(0, 256, (need + (1 << 20),), generator=gen, dtype=torch.uint8, device="cuda")
    y1 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode="fp8", workspace=ws)
    # the same workspace for another shape in between
    B = synth.random_bf16((700, K), seed=3)
    bq, sb = fq.act_quant(dev_bf16(B))
    fq.fp8_gemm(bq, sb, wq, sw, out_dtype=torch.bfloat16, mode="fp8", workspace=ws)
    y2 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode="fp8", workspace=ws)
    # arbitrary contents again (as a call that never completed could leave them)
    ws.random_(0, 256, generator=gen)
    y3 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode="fp8", workspace=ws)
    y0 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode="fp8", workspace=None)
    yb = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16, mode="fp8", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(y1.view(torch.int32), y3.view(torch.int32))
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.block_gemm(haq, hsa, hwq, hsw)
    rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    floor = scale_floor(haq, hwq, rows, cols).reshape(M, N)
    allowance = floor + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols).reshape(M, N)
    for y, out in ((y1, "f32"), (y0, "f32"), (yb, "bf16")):
        res = gemm_check(y_host(y, out), y_hat, bound, out, allowance if group_allowance_applies("fp8", out) else floor)
        assert res["violations"] == 0, (out, res)
    # split and unsplit sums differ only in fp32 rounding order: a few ulp of sum |partial * scale|
    d = np.abs(y1.cpu().numpy().astype(np.float64) - y0.cpu().numpy().astype(np.float64))
    assert np.all(d <= 2.0 ** -17 * bound + 1e-30), float(np.max(d / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("mode", ["exact", "fp8"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 576, 2048), (129, 200, 384), (64, 256, 256)])
def test_gemm_bias_epilogue(M, N, K, out, mode):
    """Bias added in fp32 before the output rounding: against the oracle's y_hat + bias
    (float64), with the one extra fp32 rounding of the addition allowed (2^-23 |y_hat + b|);
    a bf16 output must be within 1 ulp of RN_bf16(y_hat + b). Split-K shapes included."""
    A = synth.random_bf16((M, K), seed=5 * M + K)
    W = synth.random_bf16((N, K), seed=9 * N + K, std=0.02)
    bias = np.random.Generator(np.random.PCG64(N)).standard_normal(N).astype(np.float32)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    b = torch.from_numpy(bias).cuda()
    y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode, bias=b)
    y0 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode)
    y0b = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode, bias=torch.zeros_like(b))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16 if out == "bf16" else torch.int32),
                       y0b.view(torch.int16 if out == "bf16" else torch.int32)), "a zero bias changed the output"
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.block_gemm(haq, hsa, hwq, hsw)
    y_hat_b = y_hat + bias.astype(np.float64)[None, :]
    rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    allowance = scale_floor(haq, hwq, rows, cols).reshape(M, N) + 2.0 ** -23 * np.abs(y_hat_b)
    if group_allowance_applies(mode, out):
        allowance = allowance + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols).reshape(M, N)
    res = gemm_check(y_host(y, out), y_hat_b, bound, out, allowance)
    print(f"bias {M}x{N}x{K} {out} {mode}", res, flush=True)
    assert res["violations"] == 0, res


def _configs():
    names, i = [], 0
    while True:
        n = fq.lib.fp8q_gemm_config_name(i)
        if n is None:
            return names
        names.append(n.decode())
        i += 1


@pytest.mark.parametrize("M,N,K", [(300, 576, 2048), (129, 200, 1280)])
def test_gemm_every_tile_configuration(M, N, K):
    """Every tile configuration the planner can pick, forced in turn, in both contraction
    modes and with a split-K count, on ragged shapes that span several tiles."""
    from fp8_act_quant_amd import _lib as L
    A = synth.random_bf16((M, K), seed=13 * M + K)
    W = synth.random_bf16((N, K), seed=17 * N + K, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.block_gemm(haq, hsa, hwq, hsw)
    rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    floor = scale_floor(haq, hwq, rows, cols).reshape(M, N)
    fp8_allow = floor + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols).reshape(M, N)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    names = _configs()
    assert len(names) >= 8
    try:
        for c, name in enumerate(names):
            for splits in (1, 2):
                assert fq.lib.fp8q_gemm_force_config(c, splits) == L.FP8Q_OK
                for out, mode in (("bf16", "fp8"), ("f32", "fp8"), ("f32", "exact")):
                    if splits > 1 and mode == "exact":
                        continue
                    y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode, workspace=ws)
                    torch.cuda.synchronize()
                    res = gemm_check(y_host(y, out), y_hat, bound, out, fp8_allow if group_allowance_applies(mode, out) else floor)
                    print(f"config {name} splits {splits} {out} {mode}", res, flush=True)
                    assert res["violations"] == 0, (name, splits, out, mode, res)
        assert fq.lib.fp8q_gemm_force_config(len(names), 0) == L.FP8Q_ERR_SHAPE
        assert fq.lib.fp8q_gemm_force_config(0, 9) == L.FP8Q_ERR_SHAPE
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


def test_gemm_tiles_agree_bitwise():
    """Without split-K every tile configuration forms each output by the same arithmetic (the
    slices in K order, each slice partial from the same matrix-unit instructions, one fp32
    promotion FMA per slice), so all configurations must give the same bits, in each
    contraction mode; the tiles differ only in which workgroup and wave compute an output
    (and, on the exact-slice 256x256 tile, in when a block's promotion is issued)."""
    from fp8_act_quant_amd import _lib as L
    M, N, K = 300, 576, 2048
    A = synth.random_bf16((M, K), seed=31337)
    W = synth.random_bf16((N, K), seed=31338, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    try:
        for out, mode in (("f32", "exact"), ("bf16", "fp8"), ("f32", "fp8"), ("bf16", "exact")):
            first = None
            for c, name in enumerate(_configs()):
                assert fq.lib.fp8q_gemm_force_config(c, 1) == L.FP8Q_OK
                y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode, workspace=None)
                torch.cuda.synchronize()
                bits = y.view(torch.int32 if out == "f32" else torch.int16).cpu()
                if first is None:
                    first = (name, bits)
                else:
                    assert torch.equal(bits, first[1]), (name, first[0], out, mode)
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


def test_gemm_bias_every_tile_bitwise():
    """The fused bias of every tile configuration's epilogue, bit for bit: the kernel adds the
    bias row to the fp32 accumulator once, before the output rounding, so with fp32 output the
    result equals the unbiased fp32 output plus the bias in fp32, and the bf16 output equals
    that sum rounded to bf16 (round to nearest even), in both contraction modes."""
    from fp8_act_quant_amd import _lib as L
    M, N, K = 300, 576, 2048
    A = synth.random_bf16((M, K), seed=4242)
    W = synth.random_bf16((N, K), seed=4243, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    b = torch.from_numpy(np.random.Generator(np.random.PCG64(4244)).standard_normal(N).astype(np.float32)).cuda()
    try:
        for c, name in enumerate(_configs()):
            assert fq.lib.fp8q_gemm_force_config(c, 1) == L.FP8Q_OK
            for mode in ("exact", "fp8"):
                y32 = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode=mode, workspace=None)
                y32b = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32, mode=mode, workspace=None, bias=b)
                y16b = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.bfloat16, mode=mode, workspace=None, bias=b)
                torch.cuda.synchronize()
                assert torch.equal((y32 + b).view(torch.int32), y32b.view(torch.int32)), (name, mode, "fp32")
                assert torch.equal(y32b.to(torch.bfloat16).view(torch.int16), y16b.view(torch.int16)), (name, mode, "bf16")
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


@pytest.mark.parametrize("nkb", [1, 2, 3, 4, 5, 6, 7, 8, 9, 14, 15])
def test_gemm_every_tile_every_slice_count(nkb):
    """Every tile configuration at every short slice count: the K loops are unrolled by
    their stage count (and, with the register prefetch, by twice that) and end in a
    remainder of up to that many slices plus the pipeline depth, so each count from 1 to 9
    (and 14, 15) takes a different path through the remainder. FP8 products and bf16 out
    (the register-prefetch schedule's mode) and fp32 exact slices, one split."""
    from fp8_act_quant_amd import _lib as L
    M, N, K = 260, 200, 128 * nkb
    A = synth.random_bf16((M, K), seed=7919 + nkb)
    W = synth.random_bf16((N, K), seed=104729 + nkb, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.block_gemm(haq, hsa, hwq, hsw)
    rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    floor = scale_floor(haq, hwq, rows, cols).reshape(M, N)
    fp8_allow = floor + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols).reshape(M, N)
    try:
        for c, name in enumerate(_configs()):
            assert fq.lib.fp8q_gemm_force_config(c, 1) == L.FP8Q_OK
            for out, mode in (("bf16", "fp8"), ("f32", "exact")):
                y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode)
                torch.cuda.synchronize()
                res = gemm_check(y_host(y, out), y_hat, bound, out, fp8_allow if group_allowance_applies(mode, out) else floor)
                assert res["violations"] == 0, (name, nkb, out, mode, res)
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


@pytest.mark.parametrize("M,N,K", [(300, 576, 2048), (129, 200, 1280), (1000, 300, 7168), (37, 64, 384)])
def test_gemm_kmajor_scales_every_tile(M, N, K):
    """K-block-major activation scales (FP8Q_SA_KMAJOR). In the default configuration the
    output meets the bound against the oracle in both modes; every tile configuration,
    with and without split-K, gives output bit-identical to the row-major scales' (the
    scale values and every arithmetic step are the same, only where the copies read them
    differs). With ragged M the last tile's rows past M read other slices' scales in this
    layout; they feed only outputs that are never stored."""
    from fp8_act_quant_amd import _lib as L
    A = synth.random_bf16((M, K), seed=31 * M + K)
    W = synth.random_bf16((N, K), seed=37 * N + K, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    aqk, sak = fq.act_quant(dev_bf16(A), scale_layout="kmajor")
    assert torch.equal(aq.view(torch.uint8), aqk.view(torch.uint8))
    assert torch.equal(sa.view(torch.int32), sak.contiguous().view(torch.int32))
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.block_gemm(haq, hsa, hwq, hsw)
    rows, cols = np.repeat(np.arange(M), N), np.tile(np.arange(N), M)
    floor = scale_floor(haq, hwq, rows, cols).reshape(M, N)
    fp8_allow = floor + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols).reshape(M, N)
    for out, mode in (("bf16", "fp8"), ("f32", "exact")):
        y = fq.fp8_gemm(aqk, sak, wq, sw, out_dtype=TORCH_OUT[out], mode=mode)
        torch.cuda.synchronize()
        res = gemm_check(y_host(y, out), y_hat, bound, out, fp8_allow if group_allowance_applies(mode, out) else floor)
        print(f"kmajor {M}x{N}x{K} {out} {mode}", res, flush=True)
        assert res["violations"] == 0, (out, mode, res)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    bits = {"bf16": torch.int16, "f32": torch.int32}
    try:
        for c, name in enumerate(_configs()):
            for splits in (1, 2):
                assert fq.lib.fp8q_gemm_force_config(c, splits) == L.FP8Q_OK
                for out, mode in (("bf16", "fp8"), ("f32", "fp8"), ("f32", "exact")):
                    if splits > 1 and mode == "exact":
                        continue
                    yr = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode, workspace=ws)
                    yk = fq.fp8_gemm(aqk, sak, wq, sw, out_dtype=TORCH_OUT[out], mode=mode, workspace=ws)
                    torch.cuda.synchronize()
                    assert torch.equal(yr.view(bits[out]), yk.view(bits[out])), (name, splits, out, mode)
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


def test_gemm_maximum_k():
    """The largest K the ABI takes (2^24 - 128, 131071 slices) with 256-row tiles, whose
    row offsets into A reach 255 * K + K - 16, just below 2^32: forced 256x128 and 256x256 (exact
    slices, fp32 out, and FP8 products, bf16 out), plus the planner's choice
    with a split-K workspace, each against the oracle on sampled outputs that include the last
    row of the 256-row tile and the ragged last column. (The K limit itself: test_abi.)"""
    from fp8_act_quant_amd import _lib as L
    M, N, K = 256, 200, (1 << 24) - 128
    print(f"gemm maximum K {M}x{N}x{K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(14)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.bfloat16)
    aq, sa = fq.act_quant(x)
    del x
    w = torch.randn((N, K), generator=g, device="cuda", dtype=torch.bfloat16) * 0.02
    wq, sw = fq.weight_quant(w)
    del w
    torch.cuda.synchronize()
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    rng = np.random.Generator(np.random.PCG64(15))
    rows = np.concatenate([[0, 127, 128, 255, 255, 255], rng.integers(0, M, 10)]).astype(np.int64)
    cols = np.concatenate([[0, 199, 128, 0, 127, 199], rng.integers(0, N, 10)]).astype(np.int64)
    y_hat, bound = oracle.block_gemm_sampled(haq, hsa, hwq, hsw, rows, cols)
    floor = scale_floor(haq, hwq, rows, cols, chunk=4)
    fp8_allow = floor + mfma_group_allowance(haq, hsa, hwq, hsw, rows, cols, chunk=4)
    names = _configs()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    cases = [("256x128w8", "f32", "exact"), ("256x128w8", "bf16", "fp8"), ("256x256w8", "bf16", "fp8"),
             ("256x256w8", "f32", "exact"), (None, "bf16", "fp8"), (None, "f32", "exact")]
    try:
        for name, out, mode in cases:
            assert fq.lib.fp8q_gemm_force_config(names.index(name) if name else -1, 1 if name else 0) == L.FP8Q_OK
            y = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode, workspace=None if name else ws)
            torch.cuda.synchronize()
            res = gemm_check(y_host(y, out)[rows, cols], y_hat, bound, out, fp8_allow if group_allowance_applies(mode, out) else floor)
            print(f"maximum K {name or 'planner'} {out} {mode}", res, flush=True)
            assert res["violations"] == 0, (name, out, mode, res)
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


def test_gemm_kmajor_scales_large_m():
    """300007 rows, K/128 = 57: per-slice scale offsets of kb * M * 4 bytes up to 68 MB and
    a ragged last tile. Output bit-identical to the row-major scales' (whose kernel path is
    checked against the oracle above), in both modes."""
    M, N, K = 300007, 256, 128 * 57
    print(f"gemm kmajor vs row-major {M}x{N}x{K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(12)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    w = (0.02 * torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32)).to(torch.bfloat16)
    aq, sa = fq.act_quant(x)
    aqk, sak = fq.act_quant(x, scale_layout="kmajor")
    del x
    wq, sw = fq.weight_quant(w)
    for out, mode, bits in (("bf16", "fp8", torch.int16), ("f32", "exact", torch.int32)):
        yr = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode=mode)
        yk = fq.fp8_gemm(aqk, sak, wq, sw, out_dtype=TORCH_OUT[out], mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(yr.view(bits), yk.view(bits)), (out, mode)
        del yr, yk


def test_gemm_kmajor_scales_bias_and_errors():
    """The bias epilogue with K-block-major scales; scale tensors in neither layout, and
    the grouped GEMM given the flag, are rejected."""
    from fp8_act_quant_amd import _lib as L
    M, N, K = 260, 576, 1024
    A = synth.random_bf16((M, K), seed=61)
    W = synth.random_bf16((N, K), seed=62, std=0.02)
    aq, sa, wq, sw = quantise_on_gpu(A, W)
    aqk, sak = fq.act_quant(dev_bf16(A), scale_layout="kmajor")
    b = dev_f32(np.random.Generator(np.random.PCG64(63)).standard_normal(N).astype(np.float32))
    for out in ("bf16", "f32"):
        yr = fq.fp8_gemm(aq, sa, wq, sw, out_dtype=TORCH_OUT[out], mode="fp8", bias=b)
        yk = fq.fp8_gemm(aqk, sak, wq, sw, out_dtype=TORCH_OUT[out], mode="fp8", bias=b)
        torch.cuda.synchronize()
        assert torch.equal(yr.view(torch.int16 if out == "bf16" else torch.int32),
                           yk.view(torch.int16 if out == "bf16" else torch.int32))
    with pytest.raises(ValueError):
        fq.fp8_gemm(aq, torch.empty((M, 2 * (K // 128)), device="cuda")[:, ::2], wq, sw)
    with pytest.raises(ValueError):
        fq.fp8_gemm(aq, torch.empty((K // 128 * 2, M), device="cuda")[::2].t(), wq, sw)
    offs = torch.tensor([0, M], dtype=torch.int64, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    assert fq.lib.fp8_grouped_gemm(aqk.data_ptr(), sak.data_ptr(), wq.data_ptr(), sw.data_ptr(), offs.data_ptr(),
                                   y.data_ptr(), L.FP8Q_OUT_BF16 | L.FP8Q_SA_KMAJOR, 1, M, N, K,
                                   None) == L.FP8Q_ERR_DTYPE


def _plan(M, N, K, y_dtype):
    import ctypes
    c, s = ctypes.c_int(-1), ctypes.c_int(-1)
    assert fq.lib.fp8q_gemm_plan(M, N, K, y_dtype, ctypes.byref(c), ctypes.byref(s)) == 0
    return fq.lib.fp8q_gemm_config_name(c.value).decode(), s.value


@pytest.mark.parametrize("name", ["q_down", "kv_down", "kv_up", "outlier"])
def test_gemm_workload_full_size_every_output(name):
    """Each large workload at full size, in the benchmark's launch (K-block-major activation
    scales, the default contraction mode, the automatic split-K workspace): every output
    against the oracle's float64 GEMM on the same codes and scales, under the plain bound
    (fp32: 1e-5 * sum |a w|; bf16: 1 ulp of the rounded oracle, with the near-cancellation
    reading). The relative error against the unquantised product is reported on a sample."""
    wl = synth.WORKLOADS[name]
    A, W = synth.make_inputs(wl)
    print(f"gemm parity {name} M={wl.M} N={wl.N} K={wl.K} out={wl.out_dtype}", flush=True)
    aq, sak = fq.act_quant(dev_bf16(A), scale_layout="kmajor")
    wq, sw = fq.weight_quant(dev_bf16(W))
    y = fq.fp8_gemm(aq, sak, wq, sw, out_dtype=TORCH_OUT[wl.out_dtype])
    torch.cuda.synchronize()
    haq, hsa, hwq, hsw = host_codes(aq), sak.contiguous().cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    # the codes the GEMM consumed are the oracle's codes (quantiser parity)
    oaq, osa = oracle.act_quant(A)
    assert np.array_equal(haq, oaq) and np.array_equal(hsa.view(np.uint32), osa.view(np.uint32))
    del oaq, osa
    res = check_every_output(y, haq, hsa, hwq, hsw, wl.out_dtype, name)
    rows, cols = synth.sample_outputs(wl.M, wl.N, 8192, seed=1)
    yh = y_host(y, wl.out_dtype)[rows, cols]
    yv = yh if wl.out_dtype == "f32" else oracle.bf16_to_f32_array(yh)
    res["rel_err_vs_unquantised_f64"] = rel_error_vs_unquantised(yv, oracle.matmul_bf16_sampled(A, W, rows, cols))
    print(name, res, flush=True)
    assert res["n"] == wl.M * wl.N
    assert res["violations"] == 0 and res["strict_violations"] == 0, (name, res)


def test_gemm_full_size_repeat_bitwise():
    """Repeated launches at full size give identical bits, on the paths the q_down repeat
    does not take: kv_down's split-K schedule (two K ranges, partials exchanged through the
    automatic workspace), the KV up-projection's many rounds of 256x256 tiles and the outlier
    shape's exact-slice contraction. kv_down runs A1,
    then A2 through the same workspace, then A1 again: the two A1 results must be identical
    and the A2 result must meet the bound on every output."""
    g = torch.Generator(device="cuda").manual_seed(31)
    M, N, K = 4096, 576, 7168
    assert fq.gemm_workspace_bytes(M, N, K, torch.bfloat16) > 0, "kv_down expected to use split-K"
    wq, sw = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    aq1, sa1 = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16), scale_layout="kmajor")
    aq2, sa2 = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16), scale_layout="kmajor")
    y1 = fq.fp8_gemm(aq1, sa1, wq, sw).view(torch.int16)
    y2 = fq.fp8_gemm(aq2, sa2, wq, sw).view(torch.int16)
    y1b = fq.fp8_gemm(aq1, sa1, wq, sw).view(torch.int16)
    torch.cuda.synchronize()
    assert torch.equal(y1, y1b), int((y1 != y1b).sum())
    res = check_every_output(y2.view(torch.bfloat16), host_codes(aq2), sa2.contiguous().cpu().numpy(), host_codes(wq),
                             sw.cpu().numpy(), "bf16", "kv_down second input")
    assert res["violations"] == 0 and res["strict_violations"] == 0, res
    del y1, y2, y1b, aq1, aq2
    # the KV up-projection: 256x256 tiles, 16 rounds of them
    M, N, K = 8192, 32768, 512
    assert _plan(M, N, K, 1) == ("256x256w8", 1)
    aq, sa = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16), scale_layout="kmajor")
    wq, sw = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    ys = [fq.fp8_gemm(aq, sa, wq, sw).view(torch.int16) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:]), [int((ys[0] != y).sum()) for y in ys[1:]]
    del ys, aq, sa, wq, sw
    M, N, K = 16384, 7168, 7168
    aq, sa = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16), scale_layout="kmajor")
    wq, sw = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    ys = [fq.fp8_gemm(aq, sa, wq, sw, out_dtype=torch.float32).view(torch.int32) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:]), [int((ys[0] != y).sum()) for y in ys[1:]]


def test_gemm_error_paths_on_device():
    from fp8_act_quant_amd import _lib as L
    a = torch.zeros((4, 128 + 16), dtype=torch.uint8, device="cuda")
    s = torch.ones((4, 1), dtype=torch.float32, device="cuda")
    y = torch.empty((4, 8), dtype=torch.float32, device="cuda")
    g = fq.lib.fp8_block_gemm
    assert g(a.data_ptr() + 8, s.data_ptr(), a.data_ptr(), s.data_ptr(), y.data_ptr(), 0, 4, 4, 128, None, 0,
             None) == L.FP8Q_ERR_ALIGN
    assert g(a.data_ptr(), s.data_ptr(), a.data_ptr(), s.data_ptr(), y.data_ptr(), 3, 4, 4, 128, None, 0,
             None) == L.FP8Q_ERR_DTYPE
    with pytest.raises(TypeError):
        fq.fp8_gemm(dev_codes(np.zeros((4, 128), np.uint8)), dev_f32(np.ones((4, 1))),
                    dev_codes(np.zeros((4, 128), np.uint8)), dev_f32(np.ones((1, 1))), out_dtype=torch.float16)
