"""Shared test helpers: host/device marshalling and the GEMM tolerance check.

The tolerance is the one stated for the block-scaled GEMM:
  * fp32 output: |y - y_hat| <= 1e-5 * sum_k |a_k w_k| per element;
  * bf16 output: y within 1 bf16 ulp (ordered bit distance <= 1) of RN_bf16(y_hat);
    where that fails only because y_hat is close to cancellation (1e-5 * bound larger
    than half a bf16 ulp of y_hat), |y - y_hat| <= 1e-5 * bound + ulp_bf16(y_hat) is
    accepted and counted separately.
y_hat and the bound come from the CPU oracle on the same codes and scales.

Matrix-unit allowance. gfx950's FP8 MFMA (every shape, measured) adds the products of
each group of 8 consecutive k at reduced alignment precision: each product is truncated
to a multiple of 2^(E - 13), E being the binary exponent of the group's largest |product|,
before the group sums are added in fp32. `mfma_group_allowance` is the resulting bound
sum_kb |sa * sw| * sum_groups sum_k (2^(E - 13) if the product is not a multiple of it).
It is used, and reported, only where a caller explicitly asks for FP8 products with fp32
output (`group_allowance_applies`): every default-mode check and every bf16-output check is
held to the plain bound above.

fp32 scale-product floor. The kernel forms f = sa * sw in fp32 once per slice; when that
product falls below the fp32 normal range (tile and block amax both tiny) it carries an
absolute error up to 2^-150, i.e. sum_kb |P_kb| * 2^-150 on the output. `scale_floor` is
that term; it is negligible unless sa * sw < 2^-126.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def dev_bf16(a_u16: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).view(torch.bfloat16).to(device)


def dev_codes(q_u8: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q_u8)).view(torch.float8_e4m3fn).to(device)


def dev_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_codes(q: torch.Tensor) -> np.ndarray:
    return q.view(torch.uint8).cpu().numpy()


def host_bits16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def _ordered(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(np.maximum(e - 7, -133))


def gemm_check(y: np.ndarray, y_hat: np.ndarray, bound: np.ndarray, out: str, allowance=None,
               rel: float = 1e-5) -> dict:
    """y: fp32 values (out == 'f32') or bf16 bit patterns (out == 'bf16').
    Returns counts; 'violations' must be 0. `allowance` (per element, optional) is the
    matrix-unit allowance added to the bound; 'strict_violations' counts elements outside
    the plain bound. `rel` is the bound's factor on sum |a w| (1e-5 for the block-scaled
    GEMM)."""
    y_hat = np.asarray(y_hat, dtype=np.float64)
    bound = np.asarray(bound, dtype=np.float64)
    allow = np.zeros_like(y_hat) if allowance is None else np.asarray(allowance, dtype=np.float64)
    if out == "f32":
        yv = np.asarray(y, dtype=np.float32).astype(np.float64)
        err = np.abs(yv - y_hat)
        strict = ~(err <= rel * bound)
        bad = ~(err <= rel * bound + allow)
        ratio = err / np.maximum(bound, 1e-300)
        return {"n": int(y_hat.size), "violations": int(bad.sum()), "strict_violations": int(strict.sum()),
                "max_err_over_bound": float(ratio.max(initial=0))}
    yb = np.asarray(y, dtype=np.uint16)
    ref = oracle.f64_to_bf16_array(y_hat)
    dist = np.abs(_ordered(yb) - _ordered(ref))
    within_ulp = dist <= 1
    yv = oracle.bf16_to_f32_array(yb).astype(np.float64)
    err = np.abs(yv - y_hat)
    fallback = err <= rel * bound + ulp_bf16(y_hat)
    bad = ~(within_ulp | fallback | (err <= rel * bound + ulp_bf16(y_hat) + allow))
    return {"n": int(y_hat.size), "violations": int(bad.sum()),
            "strict_violations": int((~(within_ulp | fallback)).sum()),
            "beyond_1ulp_accepted": int((~within_ulp & fallback).sum()),
            "max_ulp_distance": int(dist.max(initial=0))}


def group_allowance_applies(mode: str, out: str) -> bool:
    """The matrix-unit allowance is added only for an explicit FP8-product request with fp32
    output; the default modes and bf16 output must meet the plain bound."""
    return mode == "fp8" and out == "f32"


def rel_error_vs_unquantised(y: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(np.asarray(y, dtype=np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def mfma_group_allowance(aq: np.ndarray, sa: np.ndarray, wq: np.ndarray, sw: np.ndarray,
                         rows: np.ndarray, cols: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """Per-output bound of the matrix unit's group truncation (see module docstring) at
    outputs (rows[i], cols[i]); k is grouped in aligned runs of 8."""
    dec = oracle.e4m3_decode_all()
    dec[np.isnan(dec)] = 0.0
    K = aq.shape[1]
    nkb = K // 128
    out = np.empty(rows.shape[0], dtype=np.float64)
    for s0 in range(0, rows.shape[0], chunk):
        r = rows[s0:s0 + chunk]
        c = cols[s0:s0 + chunk]
        p = dec[aq[r]] * dec[wq[c]]                      # exact products
        g = np.abs(p).reshape(len(r), K // 8, 8)
        gmax = g.max(axis=-1)
        e = np.floor(np.log2(np.where(gmax > 0, gmax, 1.0)))
        lsb = np.exp2(e - 13)[..., None]
        lost = np.where(np.mod(g, lsb) != 0, lsb, 0.0).sum(axis=-1)     # [S, K/8]
        per_slice = lost.reshape(len(r), nkb, 16).sum(axis=-1)          # [S, nkb]
        f = np.abs(sa[r].astype(np.float64) * sw[c // 128].astype(np.float64))
        out[s0:s0 + chunk] = (per_slice * f).sum(axis=-1)
    return out


def mfma_group_allowance_rowwise(aq: np.ndarray, sa: np.ndarray, bq: np.ndarray, sb: np.ndarray,
                                 rows: np.ndarray, cols: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """mfma_group_allowance for per-row scales on the second operand (sb [N, K/128])."""
    dec = oracle.e4m3_decode_all()
    dec[np.isnan(dec)] = 0.0
    K = aq.shape[1]
    nkb = K // 128
    out = np.empty(rows.shape[0], dtype=np.float64)
    for s0 in range(0, rows.shape[0], chunk):
        r = rows[s0:s0 + chunk]
        c = cols[s0:s0 + chunk]
        g = np.abs(dec[aq[r]] * dec[bq[c]]).reshape(len(r), K // 8, 8)
        gmax = g.max(axis=-1)
        e = np.floor(np.log2(np.where(gmax > 0, gmax, 1.0)))
        lsb = np.exp2(e - 13)[..., None]
        lost = np.where(np.mod(g, lsb) != 0, lsb, 0.0).sum(axis=-1)
        per_slice = lost.reshape(len(r), nkb, 16).sum(axis=-1)
        f = np.abs(sa[r].astype(np.float64) * sb[c].astype(np.float64))
        out[s0:s0 + chunk] = (per_slice * f).sum(axis=-1)
    return out


def scale_floor(aq: np.ndarray, wq: np.ndarray, rows: np.ndarray, cols: np.ndarray, chunk: int = 4096) -> np.ndarray:
    """sum_kb |P_kb| * 2^-150 at outputs (rows[i], cols[i]) (see module docstring)."""
    dec = oracle.e4m3_decode_all()
    dec[np.isnan(dec)] = 0.0
    K = aq.shape[1]
    out = np.empty(rows.shape[0], dtype=np.float64)
    for s0 in range(0, rows.shape[0], chunk):
        r = rows[s0:s0 + chunk]
        c = cols[s0:s0 + chunk]
        p = np.abs(dec[aq[r]] * dec[wq[c]]).reshape(len(r), K // 128, 128).sum(axis=-1)
        out[s0:s0 + chunk] = p.sum(axis=-1) * 2.0 ** -150
    return out


def scale_floor_rows(sa: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """Closed-form scale floor per output row, for whole-matrix checks where the per-output
    helper above is too costly: for each row m, nkb * 128 * 448^2 * 2^-150 (every |P_kb| is at
    most 128 * 448^2) if some slice's fp32 scale product sa[m, kb] * sw[r, kb] of two non-zero
    scales falls below 2^-126 (zero included), else 0. sa [M, nkb]; sw [R, nkb] (block rows, or
    the rows of a per-row scaled operand). fp32 rounding is monotone, so the smallest product of
    a slice is |sa[m, kb]| times the smallest non-zero |sw[:, kb]|."""
    sa = np.abs(np.asarray(sa, dtype=np.float32))
    sw = np.abs(np.asarray(sw, dtype=np.float32))
    nkb = sa.shape[1]
    big = np.float32(np.finfo(np.float32).max)
    min_sw = np.where(sw > 0, sw, big).min(axis=0) if sw.shape[0] else np.full(nkb, big, np.float32)
    smallest = sa * min_sw[None, :]                                   # fp32 products
    flagged = ((sa > 0) & (min_sw < big)[None, :] & (smallest < np.float32(2.0 ** -126))).any(axis=1)
    return np.where(flagged, nkb * 128 * 448.0 ** 2 * 2.0 ** -150, 0.0)


def check_every_output(y_dev, haq, hsa, hwq, hsw, out: str, label: str, chunk_rows: int = 1024,
                       rowwise: bool = False) -> dict:
    """Every output of a block-scaled GEMM result on the device against the oracle's full
    float64 GEMM (or, with rowwise, the GEMM with per-row scales on the second operand),
    computed and compared in row chunks (bounded host memory). Counts are summed over the
    chunks; one progress line per chunk."""
    M = haq.shape[0]
    floor_rows = scale_floor_rows(hsa, hsw)
    ref = oracle.rowwise_gemm if rowwise else oracle.block_gemm
    total = None
    for r0 in range(0, M, chunk_rows):
        r1 = min(r0 + chunk_rows, M)
        y_hat, bound = ref(haq[r0:r1], hsa[r0:r1], hwq, hsw)
        yc = y_dev[r0:r1]
        yh = yc.float().cpu().numpy() if out == "f32" else host_bits16(yc)
        allow = np.broadcast_to(floor_rows[r0:r1, None], y_hat.shape)
        res = gemm_check(yh, y_hat, bound, out, allow)
        if total is None:
            total = res
        else:
            for k, v in res.items():
                total[k] = max(total[k], v) if k.startswith("max") else total[k] + v
        print(f"{label} rows {r0}..{r1 - 1}: {res}", flush=True)
    return total


def bf16_linear_rel(K: int) -> float:
    """Bound factor of the bf16 GEMM (fp32 accumulation of exact bf16 products): one fp32
    rounding of the running sum per 32-product matrix-unit step along K, plus one, each at
    most 2^-24 of sum |x w| (the products themselves are exact)."""
    return (K // 32 + 1) * 2.0 ** -24


def check_bf16_linear_every_output(y_dev, x_bits: np.ndarray, w_bits: np.ndarray, out: str, label: str,
                                   bias: np.ndarray | None = None, chunk_rows: int = 1024) -> dict:
    """Every output of a bf16 GEMM result on the device against the oracle's float64 bf16
    linear (+ bias in float64, with one extra fp32 rounding of the addition allowed: it is
    counted in 'violations', not in 'strict_violations'), in row chunks."""
    M, K = x_bits.shape
    rel = bf16_linear_rel(K)
    total = None
    for r0 in range(0, M, chunk_rows):
        r1 = min(r0 + chunk_rows, M)
        y_hat, bound = oracle.matmul_bf16(x_bits[r0:r1], w_bits)
        allow = None
        if bias is not None:
            y_hat = y_hat + bias.astype(np.float64)[None, :]
            allow = 2.0 ** -23 * np.abs(y_hat)
        yc = y_dev[r0:r1]
        yh = yc.float().cpu().numpy() if out == "f32" else host_bits16(yc)
        res = gemm_check(yh, y_hat, bound, out, allow, rel=rel)
        if total is None:
            total = res
        else:
            for k, v in res.items():
                total[k] = max(total[k], v) if k.startswith("max") else total[k] + v
    print(f"{label}: {total}", flush=True)
    return total
