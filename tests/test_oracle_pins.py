"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: hand-derived values of
the E4M3 definition (tests/golden), torch's own float8_e4m3fn / bfloat16 casts (an
independent library implementation of the same formats), closed forms, exact
invariants, an integer formulation of the GEMM and lossless special cases.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_bits(x):
    return int(np.float32(x).view(np.uint32))


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


# ------------------------------------------------------------------------------ decode

def test_decode_landmarks_golden(oracle_lib):
    for lm in _load("e4m3_landmarks.json")["landmarks"]:
        code = int(lm["code"], 16)
        got = oracle.e4m3_decode(code)
        if lm["value"] == "nan":
            assert math.isnan(got), lm
        else:
            want = float.fromhex(lm["value"]) if "0x" in lm["value"] else float(lm["value"])
            assert got == want and math.copysign(1, got) == math.copysign(1, want), lm


def test_decode_structure_all_codes(oracle_lib):
    v = oracle.e4m3_decode_all()
    nan_codes = [c for c in range(256) if math.isnan(v[c])]
    assert nan_codes == [0x7F, 0xFF]
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    assert pos[0x7E] == 448.0 and pos[0x01] == 2.0 ** -9 and pos[0x08] == 2.0 ** -6
    for c in range(0x7F):
        assert v[c | 0x80] == -v[c]
        assert math.copysign(1.0, v[c | 0x80]) == -1.0
    # every finite E4M3 value is an integer multiple of 2^-9 and a bf16 value
    fin = v[~np.isnan(v)]
    assert np.all(np.mod(fin * 512.0, 1.0) == 0.0)
    assert np.all(np.float32(fin).astype(np.float64) == fin)


def test_decode_matches_torch_float8(oracle_lib):
    v = oracle.e4m3_decode_all()
    t = _torch_decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(v) & np.isnan(t)
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.all((v == t) | both_nan)
    assert np.array_equal(np.signbit(v[~both_nan]), np.signbit(t[~both_nan]))


# ------------------------------------------------------------------------------ encode

def test_encode_roundtrip_finite_codes(oracle_lib):
    v = oracle.e4m3_decode_all()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(v[c]) == c, hex(c)


def test_encode_midpoints_ties_to_even(oracle_lib):
    v = oracle.e4m3_decode_all()
    for c in range(0x7E):
        lo, hi = v[c], v[c + 1]
        mid = np.float32((lo + hi) / 2)          # 5 significant bits: exact in fp32
        assert float(mid) == (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, (hex(c), float(mid))
        assert oracle.e4m3_encode(-mid) == even | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert oracle.e4m3_encode(below) == c
        assert oracle.e4m3_encode(above) == c + 1


def test_encode_saturation_nan_and_signed_zero(oracle_lib):
    for x in [448.0, 449.0, 463.99, 464.0, 480.0, 1e30, np.inf]:
        assert oracle.e4m3_encode(x) == 0x7E
        assert oracle.e4m3_encode(-x) == 0xFE
    assert oracle.e4m3_encode(np.nan) in (0x7F, 0xFF)
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(1e-30) == 0x00
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00          # tie 0 | 2^-9 -> even (0)
    assert oracle.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01


def test_encode_matches_torch_cast_on_dense_sample(oracle_lib):
    # torch's float32 -> float8_e4m3fn cast is round-to-nearest-even; it does not
    # saturate, so compare only below the overflow threshold (464).
    top = int(np.float32(463.9).view(np.uint32))
    bits = np.arange(0, top, 97, dtype=np.uint32)            # ~11.4M patterns, all binades
    rng = np.random.Generator(np.random.PCG64(7))
    bits = np.concatenate([bits, rng.integers(0, top, size=1 << 20, dtype=np.uint32)])
    vals = bits.view(np.float32)
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(oracle.e4m3_encode_array(vals), _torch_encode(vals))


def test_encode_matches_torch_cast_near_every_midpoint(oracle_lib):
    v = oracle.e4m3_decode_all()[:0x7F]
    mids = np.float32((v[:-1] + v[1:]) / 2)
    pts = [mids]
    x = mids.copy()
    y = mids.copy()
    for _ in range(8):
        x = np.nextafter(x, np.float32(0))
        y = np.nextafter(y, np.float32(np.inf))
        pts += [x.copy(), y.copy()]
    vals = np.concatenate(pts + [np.float32(v)])
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(oracle.e4m3_encode_array(vals), _torch_encode(vals))


# ------------------------------------------------------------------------------ bf16

def test_f32_to_bf16_matches_torch(oracle_lib):
    rng = np.random.Generator(np.random.PCG64(3))
    bits = rng.integers(0, 0x7F800000, size=1 << 20, dtype=np.uint32)
    special = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x00000001, 0x00008000,
                        0x00018000, 0x3F808000, 0x3F818000, 0x00000000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_array(v), want)


# ------------------------------------------------------------------------------ act quant

def _golden_tile(spec):
    t = np.zeros(128, dtype=np.uint16)
    for i, h in spec:
        t[i] = int(h, 16)
    return t


def test_act_quant_golden_cases(oracle_lib):
    cases = _load("act_quant_cases.json")["cases"]
    x = np.stack([_golden_tile(c["tile"]) for c in cases])
    q, s = oracle.act_quant(x)
    for i, c in enumerate(cases):
        assert int(s[i, 0].view(np.uint32)) == int(c["scale_bits"], 16), c["name"]
        for idx, code in c["codes"]:
            assert q[i, idx] == int(code, 16), (c["name"], idx)


def _torch_act_quant(x_bits: np.ndarray):
    """Same steps expressed with torch CPU ops and torch's own E4M3 cast."""
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float()
    M, K = x.shape
    t = x.reshape(M, K // 128, 128)
    amax = t.abs().amax(dim=-1, keepdim=True)
    s = amax / 448.0
    d = torch.where(amax == 0, torch.ones_like(s), s)
    q = (t / d).to(torch.float8_e4m3fn).view(torch.uint8).reshape(M, K)
    return q.numpy(), s.reshape(M, K // 128).numpy()


@pytest.mark.parametrize("M,K,seed", [(37, 512, 0), (5, 128, 1), (64, 256, 2)])
def test_act_quant_matches_torch_steps(oracle_lib, M, K, seed):
    x = synth.random_bf16((M, K), seed)
    q, s = oracle.act_quant(x)
    tq, ts = _torch_act_quant(x)
    assert np.array_equal(q, tq)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))


def test_act_quant_special_tiles_match_torch_steps(oracle_lib):
    x = synth.special_tiles()
    q, s = oracle.act_quant(x)
    tq, ts = _torch_act_quant(x)
    assert np.array_equal(q, tq)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))


def test_act_quant_invariants(oracle_lib):
    x = synth.random_bf16((64, 1024), 11)
    q, s = oracle.act_quant(x)
    xf = oracle.bf16_to_f32_array(x).reshape(64, 8, 128)
    qt = q.reshape(64, 8, 128)
    amax = np.abs(xf).max(axis=-1)
    # scale: IEEE fp32 amax/448, re-derived through float64 (double rounding of a
    # quotient through 53 >= 2*24+2 bits is innocuous)
    assert np.array_equal(s, np.float32(amax.astype(np.float64) / 448.0))
    # the amax element codes to +-448
    idx = np.abs(xf).argmax(axis=-1)
    codes = np.take_along_axis(qt, idx[..., None], axis=-1)[..., 0]
    assert np.all((codes & 0x7F) == 0x7E)
    # sign of every code equals the sign bit of the input
    assert np.array_equal(qt >> 7, (x.reshape(64, 8, 128) >> 15).astype(np.uint8))
    # |decode(q) - x/s| <= half an E4M3 ulp at that magnitude
    dec = oracle.e4m3_decode_all()[qt]
    quo = xf.astype(np.float64) / s[..., None].astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(dec), 2.0 ** -6)))
    half_ulp = 2.0 ** (e - 4)
    assert np.all(np.abs(dec - quo) <= half_ulp * (1 + 1e-6))


@pytest.mark.parametrize("k", [-40, -3, 1, 7, 60])
def test_act_quant_power_of_two_invariance(oracle_lib, k):
    # Scaling a tile by 2^k (no overflow/underflow) keeps every code and scales the
    # scale by exactly 2^k.
    x = synth.random_bf16((16, 256), 5)
    xf = oracle.bf16_to_f32_array(x)
    x2 = synth.bf16_bits(np.float32(xf * np.float32(2.0 ** k)))
    assert np.array_equal(oracle.bf16_to_f32_array(x2), np.float32(xf * 2.0 ** k))
    q1, s1 = oracle.act_quant(x)
    q2, s2 = oracle.act_quant(x2)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, np.float32(s1 * np.float32(2.0 ** k)))


def test_act_quant_zero_tiles(oracle_lib):
    x = np.zeros((3, 256), dtype=np.uint16)
    x[1, 3] = 0x8000
    x[2, 130:140] = 0x8000
    q, s = oracle.act_quant(x)
    assert np.all(s == 0) and not np.any(np.signbit(s))
    assert np.array_equal(q, (x >> 8).astype(np.uint8))


# ------------------------------------------------------------------------------ weight quant

def _torch_weight_quant(w_bits: np.ndarray):
    w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).float()
    N, K = w.shape
    nnb = (N + 127) // 128
    pad = torch.zeros(nnb * 128, K)
    pad[:N] = w
    t = pad.reshape(nnb, 128, K // 128, 128)
    amax = t.abs().amax(dim=(1, 3), keepdim=True)
    s = amax / 448.0
    d = torch.where(amax == 0, torch.ones_like(s), s)
    q = (t / d).to(torch.float8_e4m3fn).view(torch.uint8).reshape(nnb * 128, K)[:N]
    return q.numpy(), s.reshape(nnb, K // 128).numpy()


@pytest.mark.parametrize("N,K", [(256, 256), (200, 384), (64, 128), (576, 256), (1, 128)])
def test_weight_quant_matches_torch_steps(oracle_lib, N, K):
    w = synth.random_bf16((N, K), N + K, std=0.02)
    q, s = oracle.weight_quant(w)
    tq, ts = _torch_weight_quant(w)
    assert s.shape == ((N + 127) // 128, K // 128)
    assert np.array_equal(q, tq)
    assert np.array_equal(s.view(np.uint32), ts.view(np.uint32))


def test_weight_quant_ragged_block_uses_valid_rows_only(oracle_lib):
    # N = 130: block row 1 has two valid rows; its amax must come from those rows.
    w = np.zeros((130, 128), dtype=np.uint16)
    w[:128] = 0x4460          # 896 in the full block
    w[128, 0] = 0x40E0        # 7.0 -> scale 2^-6 in the ragged block
    q, s = oracle.weight_quant(w)
    assert s[0, 0] == np.float32(2.0) and s[1, 0] == np.float32(2.0 ** -6)
    assert q[128, 0] == 0x7E and np.all(q[:128] == 0x7E)


def test_weight_quant_equals_act_quant_on_one_row_blocks(oracle_lib):
    # With N = 1 every 128x128 block holds a single row: the block quantiser must then
    # agree exactly with the 1x128 activation quantiser.
    x = synth.random_bf16((1, 1024), 21)
    qa, sa = oracle.act_quant(x)
    qw, sw = oracle.weight_quant(x)
    assert np.array_equal(qa, qw) and np.array_equal(sa, sw)


# ------------------------------------------------------------------------------ dequant

def test_dequant_unit_scale_is_exact_decode(oracle_lib):
    q = np.tile(np.arange(256, dtype=np.uint8), (130, 1))[:, :256]
    q[q == 0x7F] = 0
    q[q == 0xFF] = 0
    s = np.ones((2, 2), dtype=np.float32)
    w = oracle.weight_dequant(q, s)
    dec = oracle.e4m3_decode_all()[q]
    assert np.array_equal(oracle.bf16_to_f32_array(w).astype(np.float64), dec)
    assert np.array_equal(np.signbit(oracle.bf16_to_f32_array(w)), np.signbit(dec))


@pytest.mark.parametrize("N,K", [(200, 384), (576, 256)])
def test_dequant_matches_torch(oracle_lib, N, K):
    w0 = synth.random_bf16((N, K), 99, std=0.02)
    q, s = oracle.weight_quant(w0)
    w = oracle.weight_dequant(q, s)
    tq = torch.from_numpy(q).view(torch.float8_e4m3fn).float()
    ts = torch.from_numpy(s).repeat_interleave(128, 0)[:N].repeat_interleave(128, 1)
    want = (tq * ts).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(w, want)


# ------------------------------------------------------------------------------ GEMM

def test_gemm_golden_small(oracle_lib):
    g = _load("gemm_small.json")
    M, N, K = g["M"], g["N"], g["K"]

    def rows(spec):
        out = np.zeros((len(spec["rows"]), K), dtype=np.uint16)
        for i, r in enumerate(spec["rows"]):
            out[i] = int(r["fill"], 16)
            for k, h in r["set"]:
                out[i, k] = int(h, 16)
        return out

    A, W = rows(g["A"]), rows(g["W"])
    aq, sa = oracle.act_quant(A)
    wq, sw = oracle.weight_quant(W)
    assert [[hex(int(v))] for v in sa.view(np.uint32)[:, 0]] == g["sa_bits"]
    assert hex(int(sw.view(np.uint32)[0, 0])) == g["sw_bits"][0][0]
    assert np.all(wq[0] == int(g["W_codes"]["row0_all"], 16))
    assert wq[1, 0] == int(g["W_codes"]["row1_k0"], 16)
    y, b = oracle.block_gemm(aq, sa, wq, sw)
    assert np.array_equal(y, np.array(g["Y"]))
    assert np.array_equal(b, np.array(g["bound"]))


def _int_gemm(aq, sa, wq, sw):
    """Integer formulation: E4M3 codes times 2^9 are integers, so each slice partial is
    an exact int64 matmul; y = sum_kb (P_kb * 2^-18) * (sa * sw) in float64."""
    dec = oracle.e4m3_decode_all()
    dec[np.isnan(dec)] = 0
    ai = (dec[aq] * 512).astype(np.int64)
    wi = (dec[wq] * 512).astype(np.int64)
    M, K = aq.shape
    N = wq.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    nb = np.arange(N) // 128
    for kb in range(K // 128):
        sl = slice(kb * 128, (kb + 1) * 128)
        p = (ai[:, sl] @ wi[:, sl].T).astype(np.float64) * 2.0 ** -18
        f = sa[:, kb].astype(np.float64)[:, None] * sw[nb, kb].astype(np.float64)[None, :]
        y += p * f
    return y


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (33, 200, 384), (5, 576, 128)])
def test_gemm_matches_integer_formulation(oracle_lib, M, N, K):
    A = synth.random_bf16((M, K), 1)
    W = synth.random_bf16((N, K), 2, std=0.02)
    aq, sa = oracle.act_quant(A)
    wq, sw = oracle.weight_quant(W)
    y, b = oracle.block_gemm(aq, sa, wq, sw)
    assert np.array_equal(y, _int_gemm(aq, sa, wq, sw))
    # bound = sum_k |a_k w_k| over the dequantised operands (float64 matmul, own order)
    dec = oracle.e4m3_decode_all()
    ad = np.abs(dec[aq]) * np.repeat(sa.astype(np.float64), 128, axis=1)
    wd = np.abs(dec[wq]) * np.repeat(sw.astype(np.float64), 128, axis=1)[np.arange(N) // 128]
    assert np.allclose(b, ad @ wd.T, rtol=1e-12, atol=0)
    assert np.all(np.abs(y) <= b * (1 + 1e-12))


def test_gemm_sampled_equals_full(oracle_lib):
    A = synth.random_bf16((40, 256), 3)
    W = synth.random_bf16((300, 256), 4, std=0.02)
    aq, sa = oracle.act_quant(A)
    wq, sw = oracle.weight_quant(W)
    y, b = oracle.block_gemm(aq, sa, wq, sw)
    r, c = synth.sample_outputs(40, 300, 500, seed=9)
    ys, bs = oracle.block_gemm_sampled(aq, sa, wq, sw, r, c)
    assert np.array_equal(ys, y[r, c]) and np.array_equal(bs, b[r, c])


def test_gemm_one_hot_rows(oracle_lib):
    # A row with a single non-zero at k0 quantises to +-448 at k0 and zero scales
    # elsewhere, so y[n] = +-448 * sa[k0/128] * sw[n/128, k0/128] * decode(wq[n, k0]).
    M, N, K = 6, 300, 512
    A = np.zeros((M, K), dtype=np.uint16)
    ks = [0, 127, 128, 300, 383, 511]
    vals = [0x3F80, 0xC2F6, 0x0003, 0x7F7F, 0xBC00, 0x4123]
    for m, (k0, v) in enumerate(zip(ks, vals)):
        A[m, k0] = v
    W = synth.random_bf16((N, K), 8, std=0.02)
    aq, sa = oracle.act_quant(A)
    wq, sw = oracle.weight_quant(W)
    y, b = oracle.block_gemm(aq, sa, wq, sw)
    dec = oracle.e4m3_decode_all()
    for m, k0 in enumerate(ks):
        sign = -1.0 if A[m, k0] & 0x8000 else 1.0
        assert aq[m, k0] == (0xFE if sign < 0 else 0x7E)
        kb = k0 // 128
        want = (sign * 448.0 * dec[wq[:, k0]]) * (np.float64(sa[m, kb]) * sw[np.arange(N) // 128, kb].astype(np.float64))
        assert np.array_equal(y[m], want)
        assert np.array_equal(b[m], np.abs(want))


def test_gemm_lossless_inputs_equal_float64_matmul(oracle_lib):
    # Every A tile / W block is (E4M3 values) x 2^e with its max |.| = 448 * 2^e, so
    # quantisation is lossless and the block-scaled GEMM must equal the float64 matmul of
    # the original inputs exactly (exponents kept small so that matmul is exact too).
    rng = np.random.Generator(np.random.PCG64(12))
    dec = oracle.e4m3_decode_all()
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    M, N, K = 48, 260, 256
    ca = rng.choice(finite, size=(M, K))
    cw = rng.choice(finite, size=(N, K))
    ca[:, ::128] = 0x7E          # pin every tile's max to 448
    cw[::128, ::128] = 0xFE      # and every block's max to 448 (negative)
    ea = rng.integers(-2, 3, size=(M, K // 128))
    ew = rng.integers(-2, 3, size=((N + 127) // 128, K // 128))
    a64 = dec[ca] * np.repeat(2.0 ** ea, 128, axis=1)
    w64 = dec[cw] * np.repeat(2.0 ** ew, 128, axis=1)[np.arange(N) // 128]
    A = synth.bf16_bits(a64.astype(np.float32))
    W = synth.bf16_bits(w64.astype(np.float32))
    aq, sa = oracle.act_quant(A)
    wq, sw = oracle.weight_quant(W)
    assert np.array_equal(sa, np.float32(2.0 ** ea)) and np.array_equal(sw, np.float32(2.0 ** ew))
    y, _ = oracle.block_gemm(aq, sa, wq, sw)
    assert np.array_equal(y, a64 @ w64.T)


@pytest.mark.parametrize("k", [-7, 3])
def test_gemm_power_of_two_scale_linearity(oracle_lib, k):
    A = synth.random_bf16((16, 384), 13)
    W = synth.random_bf16((130, 384), 14, std=0.02)
    aq, sa = oracle.act_quant(A)
    wq, sw = oracle.weight_quant(W)
    y1, b1 = oracle.block_gemm(aq, sa, wq, sw)
    y2, b2 = oracle.block_gemm(aq, np.float32(sa * np.float32(2.0 ** k)), wq, sw)
    assert np.array_equal(y2, y1 * 2.0 ** k) and np.array_equal(b2, b1 * 2.0 ** k)


def test_gemm_single_slice_closed_form(oracle_lib):
    A = synth.random_bf16((7, 128), 15)
    W = synth.random_bf16((9, 128), 16, std=0.02)
    aq, sa = oracle.act_quant(A)
    wq, sw = oracle.weight_quant(W)
    y, _ = oracle.block_gemm(aq, sa, wq, sw)
    dec = oracle.e4m3_decode_all()
    p = dec[aq] @ dec[wq].T                       # exact: multiples of 2^-18, < 2^53
    want = p * (sa[:, 0].astype(np.float64)[:, None] * np.float64(sw[0, 0]))
    assert np.array_equal(y, want)


def test_matmul_bf16_sampled(oracle_lib):
    A = synth.random_bf16((10, 256), 17)
    W = synth.random_bf16((20, 256), 18)
    r, c = np.arange(10).repeat(20), np.tile(np.arange(20), 10)
    y = oracle.matmul_bf16_sampled(A, W, r, c)
    want = oracle.bf16_to_f32_array(A).astype(np.float64) @ oracle.bf16_to_f32_array(W).astype(np.float64).T
    assert np.allclose(y, want.reshape(-1), rtol=1e-13, atol=1e-13)


def test_matmul_bf16_small_integers_equal_integer_matmul(oracle_lib):
    """bf16 linear (the bf16 branch of linear()): on bf16 values that are small integers times
    a per-row and per-column power of two, every product and every partial sum is exact, so the
    oracle must equal the integer matrix product scaled by those powers of two (numpy int64,
    an independent routine), and its bound must equal the product of the absolute values."""
    rng = np.random.Generator(np.random.PCG64(23))
    M, N, K = 13, 37, 192
    ia = rng.integers(-15, 16, size=(M, K))
    iw = rng.integers(-15, 16, size=(N, K))
    ea = rng.integers(-6, 7, size=(M, 1))
    ew = rng.integers(-6, 7, size=(N, 1))
    A = synth.bf16_bits((ia * 2.0 ** ea).astype(np.float32))
    W = synth.bf16_bits((iw * 2.0 ** ew).astype(np.float32))
    y, b = oracle.matmul_bf16(A, W)
    scale = 2.0 ** (ea + ew.T)
    assert np.array_equal(y, (ia @ iw.T) * scale)
    assert np.array_equal(b, (np.abs(ia) @ np.abs(iw).T) * scale)


def test_matmul_bf16_one_hot_rows(oracle_lib):
    """A row of x with a single non-zero c at k0 gives y[m, n] = c * w[n, k0] exactly and a
    bound of |y| (a wrong index or transposed operand picks another element of w)."""
    M, N, K = 5, 70, 128
    W = synth.random_bf16((N, K), 29, std=0.02)
    A = np.zeros((M, K), dtype=np.uint16)
    k0 = [0, 1, 63, 64, 127]
    c = [1.0, -2.0, 0.5, 3.0, -0.25]
    for m in range(M):
        A[m, k0[m]] = synth.bf16_bits(np.float32([c[m]]))[0]
    y, b = oracle.matmul_bf16(A, W)
    w = oracle.bf16_to_f32_array(W).astype(np.float64)
    for m in range(M):
        assert np.array_equal(y[m], c[m] * w[:, k0[m]])
        assert np.array_equal(b[m], np.abs(y[m]))


def test_matmul_bf16_sampled_equals_full(oracle_lib):
    A = synth.random_bf16((9, 320), 31)
    W = synth.random_bf16((21, 320), 32, std=0.02)
    y, _ = oracle.matmul_bf16(A, W)
    r, c = np.arange(9).repeat(21), np.tile(np.arange(21), 9)
    assert np.array_equal(oracle.matmul_bf16_sampled(A, W, r, c), y.reshape(-1))


def test_f64_to_bf16_single_rounding(oracle_lib):
    # On doubles that are fp32 values, torch's float64 -> bfloat16 cast is one rounding and
    # must agree. Just off a bf16 midpoint (+- one float64 ulp) a correct single rounding
    # goes to the nearer neighbour (torch detours through fp32 there and lands on the
    # midpoint, so it is not used for those); exact midpoints go to the even pattern.
    rng = np.random.Generator(np.random.PCG64(4))
    v = (rng.standard_normal(1 << 18) * np.exp2(rng.integers(-130, 120, size=1 << 18))).astype(np.float32)
    v = np.concatenate([v, -v]).astype(np.float64)
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_array(v), want)
    b = rng.integers(0, 0x7F7F, size=4096).astype(np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    assert np.array_equal(oracle.f64_to_bf16_array(np.nextafter(mid, 0)), b.astype(np.uint16))
    assert np.array_equal(oracle.f64_to_bf16_array(np.nextafter(mid, np.inf)), (b + 1).astype(np.uint16))
    even = np.where((b & 1) == 0, b, b + 1).astype(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_array(mid), even)
    assert np.array_equal(oracle.f64_to_bf16_array(-mid), even | 0x8000)


# ----------------------------------------------------------------------------------
# Routed-expert GEMM (per-expert composition of the block GEMM) and its routing inputs
# ----------------------------------------------------------------------------------

def test_grouped_gemm_identifies_the_owning_expert(oracle_lib):
    """Closed form: A's row r holds the code of 1.0 at k = r mod 128; every entry of expert
    e's weight is the code of e + 1; unit scales. Output row r is then e + 1 for the expert
    owning r (NaN where none does): a wrong expert or boundary shows as a wrong integer."""
    K, N = 128, 5
    sizes = [3, 0, 1, 4, 0, 2]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    R = int(offsets[-1]) + 2                       # two trailing rows no expert owns
    aq = np.zeros((R, K), np.uint8)
    aq[np.arange(R), np.arange(R) % K] = 0x38      # 1.0
    sa = np.ones((R, 1), np.float32)
    one_to_six = [0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C]   # 1.0, 2.0, 3.0, 4.0, 5.0, 6.0
    E = len(sizes)
    wq = np.stack([np.full((N, K), one_to_six[e], np.uint8) for e in range(E)])
    sw = np.ones((E, 1, 1), np.float32)
    y, b = oracle.grouped_gemm(aq, sa, wq, sw, offsets)
    want = np.full(R, np.nan)
    for e in range(E):
        want[offsets[e]:offsets[e + 1]] = e + 1
    assert np.array_equal(y[:, 0], want, equal_nan=True)
    assert np.all((y == want[:, None]) | np.isnan(want)[:, None])
    # the sampled form agrees on every owned output
    rows = np.repeat(np.arange(offsets[-1]), N)
    cols = np.tile(np.arange(N), int(offsets[-1]))
    ys, bs = oracle.grouped_gemm_sampled(aq, sa, wq, sw, offsets, rows, cols)
    assert np.array_equal(ys, y[rows, cols]) and np.array_equal(bs, b[rows, cols])


def test_grouped_gemm_invariant_under_expert_relabelling(oracle_lib):
    """Swapping two experts together with their row blocks permutes the output rows the
    same way."""
    rng = np.random.Generator(np.random.PCG64(3))
    K, N = 256, 130
    sizes = [5, 7]
    aq = rng.integers(0, 256, size=(12, K), dtype=np.uint8)
    aq[(aq & 0x7F) == 0x7F] = 0
    sa = rng.uniform(0.5, 2, size=(12, 2)).astype(np.float32)
    wq = rng.integers(0, 256, size=(2, N, K), dtype=np.uint8)
    wq[(wq & 0x7F) == 0x7F] = 0
    sw = rng.uniform(0.5, 2, size=(2, 2, 2)).astype(np.float32)
    y, _ = oracle.grouped_gemm(aq, sa, wq, sw, np.array([0, 5, 12]))
    perm = np.r_[5:12, 0:5]
    y2, _ = oracle.grouped_gemm(aq[perm], sa[perm], wq[::-1].copy(), sw[::-1].copy(), np.array([0, 7, 12]))
    assert np.array_equal(y2, y[perm])


def test_moe_routing_is_a_valid_grouping():
    wl = synth.MOE_WORKLOADS["moe_down"]
    tok, offsets = synth.moe_routing(wl, seed=0)
    assert offsets[0] == 0 and offsets[-1] == len(tok) and np.all(np.diff(offsets) >= 0)
    assert len(offsets) == wl.local_experts + 1
    expert = np.searchsorted(offsets, np.arange(len(tok)), side="right") - 1
    # each token once per expert, ascending within an expert, at most top_k rows per token
    for e in range(wl.local_experts):
        t = tok[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(t) > 0)
    assert np.bincount(tok, minlength=wl.tokens).max() <= wl.top_k
    assert np.all((tok >= 0) & (tok < wl.tokens)) and np.all(expert < wl.local_experts)
    # about tokens * top_k * local / n_experts rows; expert loads vary (biased gates)
    mean = wl.tokens * wl.top_k * wl.local_experts / wl.n_experts
    assert 0.5 * mean < len(tok) < 1.5 * mean
    assert np.diff(offsets).max() > 2 * np.diff(offsets).min()
    tok2, off2 = synth.moe_routing(wl, seed=0)
    assert np.array_equal(tok, tok2) and np.array_equal(offsets, off2)


# ----------------------------------------------------------------------------------
# Training GEMMs: per-row scaled GEMM, token-wise quantisation, weight transpose
# ----------------------------------------------------------------------------------

def _finite_codes(rng, shape):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x00
    return q


def _dequant_rows(q, s_rows):
    """float64 decode(q) * s for per-row-and-slice scales s [R, K/128]."""
    dec = oracle.e4m3_decode_all()
    return dec[q] * np.repeat(s_rows.astype(np.float64), 128, axis=1)


def test_rowwise_gemm_reduces_to_block_gemm(oracle_lib):
    """With the second operand's row scales equal within each 128-row block, the per-row
    GEMM is the pinned block GEMM, bit for bit (value and bound)."""
    rng = np.random.Generator(np.random.PCG64(11))
    M, N, K = 37, 300, 384
    aq, bq = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    sa = rng.uniform(0.1, 3, size=(M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.1, 3, size=(-(-N // 128), K // 128)).astype(np.float32)
    sb = np.repeat(sw, 128, axis=0)[:N]
    y1, b1 = oracle.block_gemm(aq, sa, bq, sw)
    y2, b2 = oracle.rowwise_gemm(aq, sa, bq, sb)
    assert np.array_equal(y1, y2) and np.array_equal(b1, b2)


def test_rowwise_gemm_matches_float64_product_of_dequantised(oracle_lib):
    """Y equals the float64 matrix product of the dequantised operands (every dequantised
    value is exact in float64; only the summation order differs)."""
    rng = np.random.Generator(np.random.PCG64(12))
    M, N, K = 50, 70, 512
    aq, bq = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    sa = rng.uniform(0.01, 2, size=(M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.01, 2, size=(N, K // 128)).astype(np.float32)
    y, b = oracle.rowwise_gemm(aq, sa, bq, sb)
    ref = _dequant_rows(aq, sa) @ _dequant_rows(bq, sb).T
    assert np.all(np.abs(y - ref) <= 1e-12 * b + 1e-300)
    ys, bs = oracle.rowwise_gemm_sampled(aq, sa, bq, sb, [0, 49, 7], [0, 69, 33])
    assert np.array_equal(ys, y[[0, 49, 7], [0, 69, 33]]) and np.array_equal(bs, b[[0, 49, 7], [0, 69, 33]])


def test_rowwise_gemm_row_scale_linearity(oracle_lib):
    """Doubling the scales of one row of the second operand doubles that output column
    exactly and leaves the others unchanged."""
    rng = np.random.Generator(np.random.PCG64(13))
    M, N, K = 9, 20, 256
    aq, bq = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    sa = rng.uniform(0.1, 2, size=(M, 2)).astype(np.float32)
    sb = rng.uniform(0.1, 2, size=(N, 2)).astype(np.float32)
    y, _ = oracle.rowwise_gemm(aq, sa, bq, sb)
    sb2 = sb.copy()
    sb2[5] *= 2
    y2, _ = oracle.rowwise_gemm(aq, sa, bq, sb2)
    assert np.array_equal(y2[:, 5], 2 * y[:, 5])
    assert np.array_equal(np.delete(y2, 5, axis=1), np.delete(y, 5, axis=1))


def test_act_quant_t_closed_forms(oracle_lib):
    """Token-wise tiles with known results: a channel whose 128 tokens all equal v has scale
    RN_fp32(|v| / 448) and codes 0x7E / 0xFE; a zero channel has scale 0 and codes 0; in a
    ragged last tile only the valid tokens enter the amax and the padding is code 0."""
    M, C = 130, 16
    x = np.zeros((M, C), dtype=np.float32)
    vals = np.array([1.0, -3.5, 0.0078125, 1024.0, -0.5, 2.0 ** -20, 7.0, 0.0], dtype=np.float32)
    for c in range(8):
        x[:128, c] = vals[c]
    x[:, 8] = 1.0
    x[128, 8] = 6.0         # the ragged tile (tokens 128, 129) of channel 8: amax 6
    x[129, 8] = -3.0
    xb = synth.bf16_bits(x)
    qt, st = oracle.act_quant_t(xb)
    assert qt.shape == (C, 256) and st.shape == (C, 2)
    for c in range(8):
        v = vals[c]
        assert st[c, 0] == np.float32(abs(v)) / np.float32(448.0)
        want = 0 if v == 0 else (0x7E if v > 0 else 0xFE)
        assert np.all(qt[c, :128] == want)
    assert st[8, 1] == np.float32(6.0) / np.float32(448.0)
    assert qt[8, 128] == 0x7E and qt[8, 129] == oracle.e4m3_encode(np.float32(-3.0) / (np.float32(6.0) / np.float32(448.0)))
    assert np.all(qt[:, 130:] == 0)
    assert np.all(st[9:, :] == 0) and np.all(qt[9:, :] == 0)


def test_dgrad_through_transposed_weight_matches_dequantised_product(oracle_lib):
    """dX = dY . W through the transposed FP8 weight equals the float64 product of the
    dequantised dY (1x128 tiles along N) and dequantised W (128x128 blocks)."""
    rng = np.random.Generator(np.random.PCG64(14))
    M, N, K = 33, 256, 384
    dy = synth.random_bf16((M, N), seed=15)
    w = synth.random_bf16((N, K), seed=16, std=0.02)
    dyq, sdy = oracle.act_quant(dy)
    wq, sw = oracle.weight_quant(w)
    wqt, swt = oracle.weight_transpose(wq, sw)
    assert wqt.shape == (K, N) and swt.shape == (K // 128, N // 128)
    wq2, sw2 = oracle.weight_transpose(wqt, swt)
    assert np.array_equal(wq2, wq) and np.array_equal(sw2, sw)
    y, b = oracle.block_gemm(dyq, sdy, wqt, swt)
    dec = oracle.e4m3_decode_all()
    w_deq = dec[wq] * np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1)[:N]
    ref = _dequant_rows(dyq, sdy) @ w_deq
    assert np.all(np.abs(y - ref) <= 1e-12 * b + 1e-300)
    del rng
