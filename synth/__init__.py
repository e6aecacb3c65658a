"""Seeded synthetic inputs for FP8 block quantisation and the block-scaled GEMM.

This module only draws and enumerates inputs; it holds none of the method's
arithmetic (no amax, scale, E4M3 rounding or GEMM). Both the GPU path's tests and
the CPU oracle's tests take their inputs from here, so neither side generates data
for the other.

Recipe (one generator per workload, numpy ``Generator(PCG64(seed))``, seed 0):
  * draws are float32 standard normals, scaled in float32 (A by 1, W by 0.02),
    then rounded to bf16 with round-to-nearest-even (torch's CPU cast);
  * draw order: A, then W, then (outlier workload only) the outlier channels of A,
    then the outlier 128x128 blocks of W; both are chosen without replacement and
    multiplied in float32 before the bf16 rounding;
  * outlier counts: round(0.001 * K) channels of A scaled x100, and
    round(0.01 * #blocks) 128x128 blocks of W scaled x50.

Shapes follow the DeepSeek-V3 projections on the pomoai.com "DeepSeek-V3" page
(config_671B: dim 7168, q_lora_rank 1536, kv_lora_rank 512 plus the 64-wide rope
part; wkv_b 512 -> 128 heads x (128 + 128)).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

BLOCK = 128


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    out_dtype: str          # "f32" or "bf16"
    outliers: bool = False
    description: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 64, 256, 256, "f32", False,
                 "tiny block-scaled GEMM, A 64x256 ~N(0,1), W 256x256 ~N(0,0.02)"),
        Workload("q_down", 4096, 1536, 7168, "bf16", False,
                 "query down-projection 7168 -> 1536, 4096 tokens"),
        Workload("kv_down", 4096, 576, 7168, "bf16", False,
                 "joint KV down-projection 7168 -> 512 + 64, ragged last N-block of 64"),
        Workload("kv_up", 8192, 32768, 512, "bf16", False,
                 "KV up-projection 512 -> 128 heads x (128 + 128), 8192 latent vectors"),
        Workload("outlier", 16384, 7168, 7168, "f32", True,
                 "outlier-stress square GEMM: 0.1% of A channels x100, 1% of W blocks x50"),
    ]
}

# the workload the headline throughput figure is quoted on: the largest (1.68 TFLOP per step)
HEADLINE = "outlier"


@dataclass(frozen=True)
class MoEWorkload:
    """Routed-expert GEMM of one GPU's share of an expert-parallel MoE layer: `tokens`
    tokens each pick `top_k` of `n_experts` experts; this GPU holds experts
    0 .. local_experts-1, and multiplies the rows routed to each of them by that expert's
    [N, K] weight."""
    name: str
    tokens: int
    n_experts: int
    top_k: int
    local_experts: int
    N: int
    K: int
    out_dtype: str
    description: str = ""


MOE_WORKLOADS = {
    w.name: w
    for w in [
        MoEWorkload("moe_small", 512, 64, 6, 6, 300, 512, "bf16",
                    "small routed-expert GEMM: 6 local experts, ragged N"),
        MoEWorkload("moe_down", 8192, 256, 8, 32, 7168, 2048, "bf16",
                    "routed experts' down-projection 2048 -> 7168 (expert hidden size 2048 assumed: the pages "
                    "give none), 32 of 256 experts (one GPU of 8), 8192 tokens top-8"),
    ]
}


def moe_routing(wl: MoEWorkload, seed: int = 0):
    """Seeded top-k routing: per-token gate logits ~ N(0, 1) plus a per-expert bias
    ~ N(0, 0.5^2) (experts differ in popularity), top_k experts per token. Returns (token
    index of every row, offsets [local_experts + 1]): the rows routed to local experts,
    grouped by expert (tokens ascending within an expert)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bias = rng.standard_normal(wl.n_experts, dtype=np.float32) * np.float32(0.5)
    logits = rng.standard_normal((wl.tokens, wl.n_experts), dtype=np.float32) + bias
    top = np.argpartition(-logits, wl.top_k - 1, axis=1)[:, :wl.top_k]
    tok = np.repeat(np.arange(wl.tokens, dtype=np.int64), wl.top_k)
    exp = top.reshape(-1).astype(np.int64)
    keep = exp < wl.local_experts
    tok, exp = tok[keep], exp[keep]
    order = np.lexsort((tok, exp))
    tok, exp = tok[order], exp[order]
    counts = np.bincount(exp, minlength=wl.local_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return tok, offsets


def make_moe_inputs(wl: MoEWorkload | str, seed: int = 0):
    """(A bf16 bits [rows, K] grouped by expert, W bf16 bits [local_experts, N, K],
    offsets int64 [local_experts + 1]). Token activations ~ N(0, 1), weights ~ N(0, 0.02);
    drawn after the routing from their own generator (seed + 1), activations first."""
    if isinstance(wl, str):
        wl = MOE_WORKLOADS[wl]
    tok, offsets = moe_routing(wl, seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    x = rng.standard_normal((wl.tokens, wl.K), dtype=np.float32)
    A = bf16_bits(x[tok])
    del x
    W = np.empty((wl.local_experts, wl.N, wl.K), dtype=np.uint16)
    for e in range(wl.local_experts):
        w = rng.standard_normal((wl.N, wl.K), dtype=np.float32)
        w *= np.float32(0.02)
        W[e] = bf16_bits(w)
    return A, W, offsets


def bf16_bits(a32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_inputs(wl: Workload | str, seed: int = 0, with_weight: bool = True):
    """Return (A bf16-bits [M, K], W bf16-bits [N, K] or None) for a workload."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal((wl.M, wl.K), dtype=np.float32)
    w = None
    if with_weight or wl.outliers:
        w = rng.standard_normal((wl.N, wl.K), dtype=np.float32)
        w *= np.float32(0.02)
    if wl.outliers:
        n_ch = int(round(0.001 * wl.K))
        ch = rng.choice(wl.K, size=n_ch, replace=False)
        a[:, ch] *= np.float32(100.0)
        nnb = (wl.N + BLOCK - 1) // BLOCK
        nkb = wl.K // BLOCK
        n_blk = int(round(0.01 * nnb * nkb))
        blk = rng.choice(nnb * nkb, size=n_blk, replace=False)
        for b in blk:
            i, j = divmod(int(b), nkb)
            w[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK] *= np.float32(50.0)
    A = bf16_bits(a)
    del a
    W = bf16_bits(w) if (with_weight and w is not None) else None
    return A, W


def random_bf16(shape, seed: int, std: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return bf16_bits(a)


def sample_outputs(M: int, N: int, count: int, seed: int = 1):
    """Seeded output coordinates for sampled GEMM checks: random pairs plus the four
    corners and the first/last row and column of every 128-wide block edge."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = list(rng.integers(0, M, size=count))
    cols = list(rng.integers(0, N, size=count))
    edge_r = sorted({0, M - 1} | {min(M - 1, r) for r in range(0, M, 256)}
                    | {min(M - 1, r - 1) for r in range(256, M + 1, 256)})
    edge_c = sorted({0, N - 1} | {min(N - 1, c) for c in range(0, N, 128)}
                    | {min(N - 1, c - 1) for c in range(128, N + 1, 128)})
    for r in edge_r[:64]:
        for c in edge_c[:64]:
            rows.append(r)
            cols.append(c)
    return np.asarray(rows, dtype=np.int64), np.asarray(cols, dtype=np.int64)


# ----------------------------------------------------------------------------------
# Exhaustive enumeration of bf16 (x, amax) pairs, packed into 1x128 tiles.
# ----------------------------------------------------------------------------------
# For every positive finite bf16 magnitude pattern ab in [1, 0x7F7F] the pairs are
# all bf16 x with |x| <= value(ab), both signs. They are packed as tiles whose first
# element is +-ab (alternating sign per tile) and whose other 127 elements run through
# the sequence [0, 1, ..., ab, -0, -1, ..., -ab] (as bit patterns), zero-padded. Since
# every other element is no larger in magnitude, each tile's max |x| is value(ab).

EXHAUSTIVE_AB_MAX = 0x7F7F


def exhaustive_tile_count(ab_lo: int, ab_hi: int) -> int:
    ab = np.arange(ab_lo, ab_hi, dtype=np.int64)
    return int(((2 * (ab + 1) + 126) // 127).sum())


def exhaustive_tiles(ab_lo: int, ab_hi: int) -> np.ndarray:
    """Tiles (uint16 [T, 128]) for magnitudes ab in [ab_lo, ab_hi)."""
    ab = np.arange(ab_lo, ab_hi, dtype=np.int64)
    n_seq = 2 * (ab + 1)
    per = (n_seq + 126) // 127
    total = int(per.sum())
    starts = np.concatenate([[0], np.cumsum(per)[:-1]])
    tile_ab = np.repeat(ab, per)
    tile_j = np.arange(total, dtype=np.int64) - np.repeat(starts, per)
    out = np.zeros((total, 128), dtype=np.uint16)
    out[:, 0] = (tile_ab | ((tile_j & 1) << 15)).astype(np.uint16)
    s = tile_j[:, None] * 127 + np.arange(127, dtype=np.int64)[None, :]
    a1 = (tile_ab + 1)[:, None]
    body = np.where(s < a1, s, np.where(s < 2 * a1, 0x8000 | (s - a1), 0))
    out[:, 1:] = body.astype(np.uint16)
    return out


def exhaustive_chunks(max_tiles: int = 1 << 19):
    """Yield (ab_lo, ab_hi) ranges covering [1, 0x7F80) with at most ~max_tiles tiles each."""
    lo = 1
    end = EXHAUSTIVE_AB_MAX + 1
    while lo < end:
        # tiles for ab ~ 2*(ab+1)/127; grow the range until the budget is reached
        hi = lo
        acc = 0
        while hi < end:
            t = (2 * (hi + 1) + 126) // 127
            if acc + t > max_tiles and hi > lo:
                break
            acc += t
            hi += 1
        yield lo, hi
        lo = hi


def special_tiles() -> np.ndarray:
    """Hand-picked 1x128 tiles: all-zero, signed zeros, bf16 subnormals, the largest
    finite bf16, a single non-zero, and ties of the E4M3 rounding at scale 1."""
    tiles = []
    z = np.zeros(128, dtype=np.uint16)
    tiles.append(z.copy())                                   # all +0
    t = z.copy(); t[::2] = 0x8000; tiles.append(t)           # mixed -0 / +0
    t = np.arange(128, dtype=np.uint16); tiles.append(t)     # subnormal ramp 0..127
    t = (np.arange(128, dtype=np.uint16) | 0x8000); tiles.append(t)
    t = z.copy(); t[5] = 0x0001; tiles.append(t)             # one min subnormal
    t = z.copy(); t[0] = 0x7F7F; t[1:] = np.arange(1, 128, dtype=np.uint16) * 0x00FF
    tiles.append(t)                                          # bf16 max with spread
    t = z.copy(); t[127] = 0xFF7F; tiles.append(t)           # -max alone
    # 448 in bf16 is 0x43E0: scale 1, then every element is divided by 1 exactly
    t = z.copy(); t[0] = 0x43E0
    t[1:] = np.arange(0x3A00, 0x3A00 + 127, dtype=np.uint16)  # around 2^-11 .. 2^-10 region
    tiles.append(t)
    t = z.copy(); t[0] = 0x43E0
    t[1:] = np.arange(0x3F80, 0x3F80 + 127, dtype=np.uint16)  # [1, 2) densely: ties at 1/16
    tiles.append(t)
    return np.stack(tiles)
