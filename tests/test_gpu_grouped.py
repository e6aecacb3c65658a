"""GPU parity of the routed-expert (grouped) block-scaled GEMM against the CPU oracle,
through the C ABI.

Expert e's rows of the output are its own block-scaled GEMM, so the oracle is the pinned
block GEMM applied per expert. Small ragged groupings (empty experts, experts of one row,
of exactly one tile, of one tile plus one row) are compared on every output in both
contraction modes, and so is the routed down-projection at full size, expert by expert.
Tolerances as for the plain GEMM (tests/helpers.py).
"""
import numpy as np
import pytest
import torch

import fp8_act_quant_amd as fq
import oracle
import synth
from helpers import (check_every_output, dev_bf16, gemm_check, group_allowance_applies, host_bits16, host_codes,
                     mfma_group_allowance, scale_floor)

pytestmark = pytest.mark.gpu

TORCH_OUT = {"f32": torch.float32, "bf16": torch.bfloat16}


def y_host(y, out):
    return y.float().cpu().numpy() if out == "f32" else host_bits16(y)


def quantise_experts(A, W):
    """GPU codes of the rows [R, K] and of every expert's weight [E, N, K]."""
    aq, sa = fq.act_quant(dev_bf16(A))
    E, N, K = W.shape
    wq, sw = fq.weight_quant(dev_bf16(W.reshape(E * N, K)))
    if N % 128 == 0:
        return aq, sa, wq.view(E, N, K), sw.view(E, N // 128, K // 128)
    # a weight whose N is not a multiple of 128 has its own last scale row per expert
    qs, ss = zip(*(fq.weight_quant(dev_bf16(W[e])) for e in range(E)))
    return aq, sa, torch.stack(qs).contiguous(), torch.stack(ss).contiguous()


def allowances(haq, hsa, hwq, hsw, offsets, rows, cols, fp8_products):
    """Per-output allowance: the scale floor, plus the matrix unit's group truncation where
    an explicit FP8-product request has fp32 output, each taken against the weight of the
    expert owning the row."""
    expert = np.searchsorted(offsets, rows, side="right") - 1
    out = np.zeros(rows.shape, dtype=np.float64)
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        out[sel] = scale_floor(haq, hwq[e], rows[sel], cols[sel])
        if fp8_products:
            out[sel] += mfma_group_allowance(haq, hsa, hwq[e], hsw[e], rows[sel], cols[sel])
    return out


def offsets_of(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


@pytest.mark.parametrize("mode", ["exact", "fp8"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("sizes,N,K", [
    ([0, 1, 127, 128, 129, 0, 300, 5], 256, 256),
    ([37, 0, 0, 200], 200, 384),
    ([3, 250, 1], 1100, 128),
    ([0, 0, 64], 64, 1024),
])
def test_grouped_small_full_output(sizes, N, K, out, mode):
    E = len(sizes)
    offsets = offsets_of(sizes)
    R = int(offsets[-1])
    A = synth.random_bf16((R, K), seed=R + N + K)
    W = synth.random_bf16((E, N, K), seed=E * N + K, std=0.02)
    aq, sa, wq, sw = quantise_experts(A, W)
    off = torch.from_numpy(offsets).cuda()
    y = fq.fp8_grouped_gemm(aq, sa, wq, sw, off, out_dtype=TORCH_OUT[out], mode=mode)
    torch.cuda.synchronize()
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.grouped_gemm(haq, hsa, hwq, hsw, offsets)
    rows, cols = np.repeat(np.arange(R), N), np.tile(np.arange(N), R)
    allow = allowances(haq, hsa, hwq, hsw, offsets, rows, cols, group_allowance_applies(mode, out)).reshape(R, N)
    res = gemm_check(y_host(y, out), y_hat, bound, out, allow)
    print(f"grouped {sizes} N={N} K={K} {out} {mode}", res, flush=True)
    assert res["violations"] == 0, res


@pytest.mark.parametrize("E", [1024, 1000])
def test_grouped_maximum_expert_count(E):
    """The largest expert count the ABI takes (1024) and a count that is not a power of two:
    the device-side scan of the per-expert tile counts (several experts per thread) and the
    search for each tile's expert, with nearly every expert empty and rows at the first, two
    middle and the last expert; every output against the oracle in both default modes."""
    sizes = np.zeros(E, dtype=np.int64)
    sizes[0], sizes[E // 2], sizes[(2 * E) // 3], sizes[E - 1] = 5, 130, 1, 3
    N, K = 128, 256
    offsets = offsets_of(sizes)
    R = int(offsets[-1])
    A = synth.random_bf16((R, K), seed=E + 1)
    W = synth.random_bf16((E, N, K), seed=E + 2, std=0.02)
    aq, sa, wq, sw = quantise_experts(A, W)
    off = torch.from_numpy(offsets).cuda()
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    y_hat, bound = oracle.grouped_gemm(haq, hsa, hwq, hsw, offsets)
    rows, cols = np.repeat(np.arange(R), N), np.tile(np.arange(N), R)
    for out, mode in (("bf16", "fp8"), ("f32", "exact")):
        y = fq.fp8_grouped_gemm(aq, sa, wq, sw, off, out_dtype=TORCH_OUT[out], mode=mode)
        torch.cuda.synchronize()
        allow = allowances(haq, hsa, hwq, hsw, offsets, rows, cols, group_allowance_applies(mode, out)).reshape(R, N)
        res = gemm_check(y_host(y, out), y_hat, bound, out, allow)
        print(f"grouped E={E} {out} {mode}", res, flush=True)
        assert res["violations"] == 0, res


@pytest.mark.parametrize("out,mode,config", [("bf16", "fp8", "128x256w8"), ("f32", "fp8", "128x256w8"),
                                             ("bf16", "fp8", "128x192w8"), ("f32", "exact", "128x192w8")])
def test_grouped_bitwise_equals_per_expert_gemm(out, mode, config):
    """The grouped launch runs the same tile code as the plain GEMM: each expert's rows equal,
    bit for bit, the plain GEMM of those rows with the tile configuration the grouped
    kernel uses for this N and mode (forced, no split-K)."""
    sizes = [130, 0, 1, 255, 64]
    N = 1024 if config == "128x256w8" else 576
    K = 512
    E = len(sizes)
    offsets = offsets_of(sizes)
    R = int(offsets[-1])
    A = synth.random_bf16((R, K), seed=71)
    W = synth.random_bf16((E, N, K), seed=72, std=0.02)
    aq, sa, wq, sw = quantise_experts(A, W)
    y = fq.fp8_grouped_gemm(aq, sa, wq, sw, torch.from_numpy(offsets).cuda(), out_dtype=TORCH_OUT[out], mode=mode)
    names = []
    while (n := fq.lib.fp8q_gemm_config_name(len(names))) is not None:
        names.append(n.decode())
    try:
        assert fq.lib.fp8q_gemm_force_config(names.index(config), 1) == 0
        for e in range(E):
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 == r0:
                continue
            ye = fq.fp8_gemm(aq[r0:r1], sa[r0:r1], wq[e], sw[e], out_dtype=TORCH_OUT[out], mode=mode, workspace=None)
            iv = torch.int16 if out == "bf16" else torch.int32
            assert torch.equal(y[r0:r1].view(iv), ye.view(iv)), (e, r0, r1)
    finally:
        fq.lib.fp8q_gemm_force_config(-1, 0)


def test_grouped_rows_outside_every_expert_untouched():
    """offsets[E] < rows: the trailing rows belong to no expert and keep what `out` held;
    offsets past rows are clamped (the last expert keeps only rows it can own)."""
    K, N = 256, 320
    R = 300
    A = synth.random_bf16((R, K), seed=5)
    W = synth.random_bf16((2, N, K), seed=6, std=0.02)
    aq, sa, wq, sw = quantise_experts(A, W)
    haq, hsa, hwq, hsw = host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy()
    sentinel = torch.full((R, N), 7.0, dtype=torch.float32, device="cuda")
    offsets = np.array([0, 100, 250], dtype=np.int64)
    y = fq.fp8_grouped_gemm(aq, sa, wq, sw, torch.from_numpy(offsets).cuda(), out_dtype=torch.float32,
                            out=sentinel.clone(), mode="exact")
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(yh[250:] == 7.0)
    y_hat, bound = oracle.grouped_gemm(haq, hsa, hwq, hsw, offsets)
    rows, cols = np.repeat(np.arange(250), N), np.tile(np.arange(N), 250)
    allow = allowances(haq, hsa, hwq, hsw, offsets, rows, cols, False).reshape(250, N)
    res = gemm_check(yh[:250], y_hat[:250], bound[:250], "f32", allow)
    assert res["violations"] == 0, res
    # clamped: offsets [0, 100, 1000] over 300 rows is [0, 100, 300]
    y2 = fq.fp8_grouped_gemm(aq, sa, wq, sw, torch.tensor([0, 100, 1000], device="cuda"), out_dtype=torch.float32,
                             mode="exact")
    y3 = fq.fp8_grouped_gemm(aq, sa, wq, sw, torch.tensor([0, 100, 300], device="cuda"), out_dtype=torch.float32,
                             mode="exact")
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int32), y3.view(torch.int32))


def test_grouped_k_zero_writes_zeros():
    R, N, E = 50, 40, 3
    aq = torch.empty((R, 0), dtype=torch.float8_e4m3fn, device="cuda")
    sa = torch.empty((R, 0), dtype=torch.float32, device="cuda")
    wq = torch.empty((E, N, 0), dtype=torch.float8_e4m3fn, device="cuda")
    sw = torch.empty((E, 1, 0), dtype=torch.float32, device="cuda")
    y = fq.fp8_grouped_gemm(aq, sa, wq, sw, torch.tensor([0, 10, 10, 50], device="cuda"), out_dtype=torch.float32,
                            out=torch.full((R, N), 3.0, device="cuda"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


def test_grouped_moe_down_full_size_every_output():
    """The routed down-projection at full size: every output row of every expert against
    the oracle's block GEMM with that expert's weight, under the plain bf16 bound."""
    wl = synth.MOE_WORKLOADS["moe_down"]
    A, W, offsets = synth.make_moe_inputs(wl)
    R = int(offsets[-1])
    print(f"grouped parity moe_down rows={R} experts={wl.local_experts} N={wl.N} K={wl.K} "
          f"sizes {np.diff(offsets).min()}..{np.diff(offsets).max()}", flush=True)
    aq, sa, wq, sw = quantise_experts(A, W)
    y = fq.fp8_grouped_gemm(aq, sa, wq, sw, torch.from_numpy(offsets).cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    haq, hsa = host_codes(aq), sa.cpu().numpy()
    oaq, osa = oracle.act_quant(A)
    assert np.array_equal(haq, oaq) and np.array_equal(hsa.view(np.uint32), osa.view(np.uint32))
    # expert 0's weight codes are the oracle's (quantiser parity on one expert at full size)
    owq, osw = oracle.weight_quant(W[0])
    assert np.array_equal(host_codes(wq[0]), owq) and np.array_equal(sw[0].cpu().numpy().view(np.uint32),
                                                                     osw.view(np.uint32))
    hwq, hsw = host_codes(wq), sw.cpu().numpy()
    checked = 0
    for e in range(wl.local_experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        res = check_every_output(y[r0:r1], haq[r0:r1], hsa[r0:r1], hwq[e], hsw[e], "bf16", f"moe_down expert {e}",
                                 chunk_rows=4096)
        assert res["violations"] == 0 and res["strict_violations"] == 0, (e, res)
        checked += res["n"]
    assert checked == R * wl.N
    assert torch.isfinite(y.float()).all()


def test_grouped_error_paths():
    from fp8_act_quant_amd import _lib as L
    g = fq.lib.fp8_grouped_gemm
    a = torch.zeros((4, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones((4, 1), dtype=torch.float32, device="cuda")
    w = torch.zeros((2, 8, 128), dtype=torch.uint8, device="cuda")
    ws = torch.ones((2, 1, 1), dtype=torch.float32, device="cuda")
    off = torch.tensor([0, 2, 4, 0], dtype=torch.int64, device="cuda")
    y = torch.empty((4, 8), dtype=torch.float32, device="cuda")
    args = lambda **k: dict(dict(aq=a.data_ptr(), sa=s.data_ptr(), wq=w.data_ptr(), sw=ws.data_ptr(),
                                 off=off.data_ptr(), y=y.data_ptr(), dt=0, E=2, R=4, N=8, K=128), **k)

    def call(**k):
        v = args(**k)
        return g(v["aq"], v["sa"], v["wq"], v["sw"], v["off"], v["y"], v["dt"], v["E"], v["R"], v["N"], v["K"], None)

    assert call() == L.FP8Q_OK
    torch.cuda.synchronize()
    assert call(E=0) == L.FP8Q_ERR_SHAPE
    assert call(E=1025) == L.FP8Q_ERR_SHAPE
    assert call(K=100) == L.FP8Q_ERR_SHAPE
    assert call(off=None) == L.FP8Q_ERR_NULL
    assert call(off=off.data_ptr() + 4) == L.FP8Q_ERR_ALIGN
    assert call(dt=3) == L.FP8Q_ERR_DTYPE
    assert call(R=0) == L.FP8Q_OK
    with pytest.raises(ValueError):
        fq.fp8_grouped_gemm(a.view(torch.float8_e4m3fn), s, w.view(torch.float8_e4m3fn), ws, off[:2])
    with pytest.raises(TypeError):
        fq.fp8_grouped_gemm(a.view(torch.float8_e4m3fn), s, w.view(torch.float8_e4m3fn), ws, off[:3].int())


def test_grouped_and_plain_repeat_bitwise_at_full_size():
    """Repeated launches give identical bits (no race between the copies into a stage buffer
    and the reads of it): the routed down-projection with every local expert, and the plain
    GEMM on the q_down shape, each run three times on the same inputs."""
    wl = synth.MOE_WORKLOADS["moe_down"]
    _, offsets = synth.moe_routing(wl)
    R, E, N, K = int(offsets[-1]), wl.local_experts, wl.N, wl.K
    g = torch.Generator(device="cuda").manual_seed(5)
    aq, sa = fq.act_quant(torch.randn((R, K), generator=g, device="cuda").to(torch.bfloat16))
    wq = torch.empty((E, N, K), dtype=torch.float8_e4m3fn, device="cuda")
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for e in range(E):
        wq[e], sw[e] = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    off = torch.from_numpy(offsets).cuda()
    ys = [fq.fp8_grouped_gemm(aq, sa, wq, sw, off).view(torch.int16) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:]), [int((ys[0] != y).sum()) for y in ys[1:]]
    M, N, K = 4096, 1536, 7168
    aq, sa = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16))
    wq, sw = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    ys = [fq.fp8_gemm(aq, sa, wq, sw).view(torch.int16) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:]), [int((ys[0] != y).sum()) for y in ys[1:]]
