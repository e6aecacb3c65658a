"""fp8_block_gemm_noalloc: the block-scaled GEMM with the library's static split-K scratch
instead of a caller's workspace (for callers that cannot allocate). Through the C ABI, its
output must equal fp8_block_gemm's with a workspace of fp8_block_gemm_workspace_bytes()
(same tile and split plan, so bit for bit) and meet the oracle's bound, on two calls in a
row, the second with a smaller input; a shape whose plan needs more scratch than the static
array holds is refused before anything is enqueued."""
import pytest
import torch

import fp8_act_quant_amd as fq
from fp8_act_quant_amd import _lib as L
from helpers import check_every_output, host_codes

pytestmark = pytest.mark.gpu


def _noalloc(aq, sa, wq, sw, y, code, M, N, K):
    return fq.lib.fp8_block_gemm_noalloc(aq.data_ptr(), sa.data_ptr(), wq.data_ptr(), sw.data_ptr(), y.data_ptr(),
                                         code, M, N, K, torch.cuda.current_stream().cuda_stream)


def _with_workspace(aq, sa, wq, sw, y, code, M, N, K):
    need = int(fq.lib.fp8_block_gemm_workspace_bytes(M, N, K, code))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    st = fq.lib.fp8_block_gemm(aq.data_ptr(), sa.data_ptr(), wq.data_ptr(), sw.data_ptr(), y.data_ptr(), code, M, N,
                               K, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    return st, need, ws


@pytest.mark.parametrize("out", ["bf16", "f32_fp8_products"])
def test_noalloc_matches_workspace_entry_point_twice(out):
    """Two calls in a row, both on split-K plans that use the scratch: the joint KV
    down-projection (4096 x 576 x 7168: 96 tiles in two K ranges), then a smaller ragged shape
    (300 x 200 x 1280); each bitwise against fp8_block_gemm with its own workspace, and (bf16
    output, the default contraction) against the oracle on every output."""
    g = torch.Generator(device="cuda").manual_seed(77)
    if out == "bf16":
        code, dt, bits = L.FP8Q_OUT_BF16, torch.bfloat16, torch.int16
    else:
        code, dt, bits = L.FP8Q_OUT_F32 | L.FP8Q_GEMM_FP8_PRODUCTS, torch.float32, torch.int32
    for M, N, K in ((4096, 576, 7168), (300, 200, 1280)):
        need = int(fq.lib.fp8_block_gemm_workspace_bytes(M, N, K, code))
        print(f"noalloc {out} {M}x{N}x{K} scratch need {need}", flush=True)
        assert 0 < need <= L.FP8Q_NOALLOC_SCRATCH_BYTES
        aq, sa = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16))
        wq, sw = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
        y_na = torch.full((M, N), 7.0, dtype=dt, device="cuda")
        y_ws = torch.empty((M, N), dtype=dt, device="cuda")
        assert _noalloc(aq, sa, wq, sw, y_na, code, M, N, K) == L.FP8Q_OK
        st, _, ws = _with_workspace(aq, sa, wq, sw, y_ws, code, M, N, K)
        assert st == L.FP8Q_OK
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(bits), y_ws.view(bits)), int((y_na.view(bits) != y_ws.view(bits)).sum())
        if out == "bf16":
            res = check_every_output(y_na, host_codes(aq), sa.cpu().numpy(), host_codes(wq), sw.cpu().numpy(),
                                     "bf16", f"noalloc {M}x{N}x{K}")
            assert res["violations"] == 0 and res["strict_violations"] == 0, res
        del ws


def test_noalloc_kmajor_and_modes():
    """K-block-major activation scales and both explicit contraction modes, bitwise against
    fp8_block_gemm with a workspace."""
    g = torch.Generator(device="cuda").manual_seed(78)
    M, N, K = 1000, 576, 4096
    x = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    aq, sak = fq.act_quant(x, scale_layout="kmajor")
    wq, sw = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    for code, dt, bits in ((L.FP8Q_OUT_BF16 | L.FP8Q_GEMM_FP8_PRODUCTS, torch.bfloat16, torch.int16),
                           (L.FP8Q_OUT_F32 | L.FP8Q_GEMM_EXACT_SLICES, torch.float32, torch.int32),
                           (L.FP8Q_OUT_F32 | L.FP8Q_GEMM_FP8_PRODUCTS, torch.float32, torch.int32)):
        code |= L.FP8Q_SA_KMAJOR
        y_na = torch.empty((M, N), dtype=dt, device="cuda")
        y_ws = torch.empty((M, N), dtype=dt, device="cuda")
        assert _noalloc(aq, sak, wq, sw, y_na, code, M, N, K) == L.FP8Q_OK
        st, _, ws = _with_workspace(aq, sak, wq, sw, y_ws, code, M, N, K)
        assert st == L.FP8Q_OK
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(bits), y_ws.view(bits)), hex(code)


def test_noalloc_refuses_plans_beyond_the_scratch():
    """A shape whose split-K plan needs more than the static scratch is refused with
    FP8Q_ERR_WORKSPACE before any launch (the pointers are never dereferenced); empty shapes
    are accepted as no-ops."""
    M, N, K = 4096, 18432, 16384
    need = int(fq.lib.fp8_block_gemm_workspace_bytes(M, N, K, L.FP8Q_OUT_BF16))
    assert need > L.FP8Q_NOALLOC_SCRATCH_BYTES
    t = torch.empty(256, dtype=torch.uint8, device="cuda")
    p = t.data_ptr()
    st = fq.lib.fp8_block_gemm_noalloc(p, p, p, p, p, L.FP8Q_OUT_BF16, M, N, K, None)
    assert st == L.FP8Q_ERR_WORKSPACE
    assert "scratch" in L.strerror(st)
    assert fq.lib.fp8_block_gemm_noalloc(None, None, None, None, None, L.FP8Q_OUT_BF16, 0, N, K, None) == L.FP8Q_OK
    assert fq.lib.fp8_block_gemm_noalloc(p, p, p, p, p, 3, 4, 4, 128, None) == L.FP8Q_ERR_DTYPE
    assert fq.lib.fp8_block_gemm_noalloc(p, p, p, p, p, L.FP8Q_OUT_BF16, 4, 4, 100, None) == L.FP8Q_ERR_SHAPE


def test_noalloc_replays_in_a_captured_graph():
    """The callers this entry point is for include code under HIP graph capture: captured once
    (its split-K epoch is fixed at capture), the call is replayed three times with new
    activations copied into the captured input between replays, with eager work and
    synchronisation in between; every replay equals fp8_block_gemm with a workspace on the same
    input, bit for bit."""
    g = torch.Generator(device="cuda").manual_seed(79)
    M, N, K = 4096, 576, 7168
    code = L.FP8Q_OUT_BF16
    assert 0 < int(fq.lib.fp8_block_gemm_workspace_bytes(M, N, K, code)) <= L.FP8Q_NOALLOC_SCRATCH_BYTES
    wq, sw = fq.weight_quant((torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    aq, sa = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    # warm up on the capture stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert _noalloc(aq, sa, wq, sw, y, code, M, N, K) == L.FP8Q_OK
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert _noalloc(aq, sa, wq, sw, y, code, M, N, K) == L.FP8Q_OK
    for r in range(3):
        aq2, sa2 = fq.act_quant(torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16))
        aq.copy_(aq2)
        sa.copy_(sa2)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(y)
        st, _, ws = _with_workspace(aq, sa, wq, sw, ref, code, M, N, K)
        assert st == L.FP8Q_OK
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), (r, int((y != ref).sum()))
        del ws
