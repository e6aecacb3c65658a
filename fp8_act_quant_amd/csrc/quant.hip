// quant.hip -- E4M3 quantisation / dequantisation kernels for gfx950.
//
// act_quant: per token per 128 channels (pomoai.com "DeepSeek-V3", FP8 mixed-precision
// training section: dynamic activation quantisation per token per 128 channels).
// weight_quant / weight_dequant: 128x128 blocks with one fp32 scale each (same section:
// FP8 weights in 128x128 blocks with a float32 weight_scale_inv per block).
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

// ------------------------------------------------------------------------------------
// act_quant
// A row-major [M, K] activation with K % 128 == 0 is a flat sequence of 1x128 tiles,
// and tile t's scale is s[t] (the [M, K/128] scale grid in row-major order). One DPP row
// (16 lanes) owns a tile: lane j holds bf16 elements 8j..8j+7 (one 16-byte load) and
// writes their 8 codes (one 8-byte store). A wave covers 4 consecutive tiles per load
// instruction (1 KiB contiguous); a workgroup processes groups of AQ_TILES_PER_GROUP
// consecutive tiles, grid-stride, and issues the loads of its next group before
// quantising the current one, so that two groups' loads per lane are in flight and the
// stream never drains between groups.
// The K-block-major variant writes the scale of row m, K slice kb to s[kb * M + m] (the
// layout in which one K slice's scales of consecutive tokens are contiguous). Its groups
// are 64 consecutive rows of one K slice instead (group g: rows 64 (g / nkb) .., slice
// g % nkb), so that the four tiles of a load instruction are four consecutive rows and
// each instruction's scale stores fill 16 contiguous bytes; every tile is still one
// 256-byte run of x. The quotient g / nkb is formed by multiplication with a precomputed
// reciprocal (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994, the round-up method for unsigned N-bit division), exact for every
// 32-bit g.
// ------------------------------------------------------------------------------------
constexpr int AQ_THREADS = 256;
constexpr int AQ_UNROLL = 4;
constexpr int AQ_TILES_PER_WAVE = 4 * AQ_UNROLL;
constexpr int AQ_TILES_PER_GROUP = AQ_TILES_PER_WAVE * (AQ_THREADS / 64);

// Unsigned 32-bit division by an invariant d >= 1: with l = ceil(log2 d),
// magic = floor(2^32 (2^l - d) / d) + 1, t1 = hi32(magic * n), the quotient is
// (t1 + ((n - t1) >> min(l, 1))) >> max(l - 1, 0).
struct DivU32 {
    uint32_t d, magic;
    int sh1, sh2;
    __device__ __forceinline__ uint32_t div(uint32_t n) const {
        const uint32_t t1 = __umulhi(magic, n);
        return (t1 + ((n - t1) >> sh1)) >> sh2;
    }
};

static DivU32 make_div(uint32_t d) {
    int l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    DivU32 r;
    r.d = d;
    r.magic = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    r.sh1 = l < 1 ? l : 1;
    r.sh2 = l > 1 ? l - 1 : 0;
    return r;
}

// The AQ_UNROLL tiles of one lane in group g: tile t0 + u * step (u = 0 .. AQ_UNROLL-1),
// which exists while idx0 + 4 u < lim. Row-major: 64 consecutive flat tiles (idx = tile
// number). K-block-major: 64 consecutive rows of one K slice (idx = row, the scale goes
// to s[kb * M + row]).
struct AqLane {
    int64_t t0, step, idx0, lim, s0;   // s0: scale index of the first tile (its step is 4)
};

template <int KMAJOR>
__device__ __forceinline__ AqLane aq_lane(int64_t g, int64_t my, int64_t n_tiles, int64_t M, const DivU32 &by_nkb) {
    AqLane r;
    if constexpr (KMAJOR) {
        const int64_t nkb = by_nkb.d;
        const int64_t mb = by_nkb.div((uint32_t)g), kb = g - mb * nkb;
        const int64_t m0 = mb * AQ_TILES_PER_GROUP + my;
        r.t0 = m0 * nkb + kb;
        r.step = 4 * nkb;
        r.idx0 = m0;
        r.lim = M;
        r.s0 = kb * M + m0;
    } else {
        r.t0 = g * AQ_TILES_PER_GROUP + my;
        r.step = 4;
        r.idx0 = r.t0;
        r.lim = n_tiles;
        r.s0 = r.t0;
    }
    return r;
}

__device__ __forceinline__ void aq_load(const u32x4 *__restrict__ x, const AqLane &l, int j, bool any,
                                        u32x4 (&v)[AQ_UNROLL]) {
#pragma unroll
    for (int u = 0; u < AQ_UNROLL; ++u) {
        const int64_t t = l.t0 + u * l.step;
        v[u] = (any && l.idx0 + 4 * u < l.lim) ? __builtin_nontemporal_load(&x[t * 16 + j]) : u32x4{0, 0, 0, 0};
    }
}

// KMAJOR: scales K-block-major (s[kb * M + m]); the group count is below 2^32 there
template <int KMAJOR>
__global__ __launch_bounds__(AQ_THREADS) void act_quant_kernel(const u32x4 *__restrict__ x,
                                                               u32x2 *__restrict__ q,
                                                               float *__restrict__ s,
                                                               int64_t n_tiles, DivU32 by_nkb, int64_t M) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int64_t my = wave * AQ_TILES_PER_WAVE + (lane >> 4);   // this lane's first tile within a group
    const int64_t n_groups = KMAJOR ? (M + AQ_TILES_PER_GROUP - 1) / AQ_TILES_PER_GROUP * by_nkb.d
                                    : (n_tiles + AQ_TILES_PER_GROUP - 1) / AQ_TILES_PER_GROUP;

    int64_t g = blockIdx.x;
    u32x4 v[AQ_UNROLL];
    AqLane cur = aq_lane<KMAJOR>(g, my, n_tiles, M, by_nkb);
    aq_load(x, cur, j, g < n_groups, v);
    while (g < n_groups) {
        const int64_t gn = g + gridDim.x;
        const AqLane nxt = aq_lane<KMAJOR>(gn < n_groups ? gn : g, my, n_tiles, M, by_nkb);
        u32x4 vn[AQ_UNROLL];
        aq_load(x, nxt, j, gn < n_groups, vn);
#pragma unroll
        for (int u = 0; u < AQ_UNROLL; ++u) {
            const int64_t t = cur.t0 + u * cur.step;
            const uint32_t amax = row16_max(absmax_bits8(v[u]));
            const TileScale ts = tile_scale(amax);
            const u32x2 codes = quant8(v[u], ts);
            if (cur.idx0 + 4 * u < cur.lim) {
                // an ordinary (cache-allocating) store: the codes (1 B per element) are read
                // by the GEMM right after, and staying in the 256 MB MALL saves it the HBM
                // round trip (measured: GEMM -8%, act_quant +5%, step -2.4%); the bf16 input
                // is streamed with non-temporal loads
                q[t * 16 + j] = codes;
                if (j == 0) s[cur.s0 + 4 * u] = ts.s;
            }
        }
#pragma unroll
        for (int u = 0; u < AQ_UNROLL; ++u) v[u] = vn[u];
        cur = nxt;
        g = gn;
    }
}

// workgroups per CU of the grid-stride launch (tuning override FP8Q_AQ_WGS_PER_CU)
static int aq_wgs_per_cu() {
    static const int v = [] {
        const char *e = std::getenv("FP8Q_AQ_WGS_PER_CU");
        const int n = e ? std::atoi(e) : 0;
        return n >= 1 && n <= 32 ? n : 16;
    }();
    return v;
}

hipError_t launch_act_quant(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K, bool kmajor,
                            hipStream_t stream) {
    const int64_t n_tiles = M * (K / kBlock);
    if (n_tiles == 0) return hipSuccess;
    // (K-block-major groups: 64 rows of one K slice, numbered below 2^32)
    const int64_t groups = kmajor ? (M + AQ_TILES_PER_GROUP - 1) / AQ_TILES_PER_GROUP * (K / kBlock)
                                  : (n_tiles + AQ_TILES_PER_GROUP - 1) / AQ_TILES_PER_GROUP;
    if (kmajor && groups > 0xFFFFFFFFll) return hipErrorInvalidValue;
    const int64_t cap = (int64_t)256 * aq_wgs_per_cu();
    const int64_t blocks = groups < cap ? groups : cap;
    const DivU32 by_nkb = make_div(kmajor ? (uint32_t)(K / kBlock) : 1u);   // (unused in row-major order)
    if (kmajor)
        hipLaunchKernelGGL(act_quant_kernel<1>, dim3((unsigned)blocks), dim3(AQ_THREADS), 0, stream,
                           reinterpret_cast<const u32x4 *>(x), reinterpret_cast<u32x2 *>(q), s, n_tiles, by_nkb, M);
    else
        hipLaunchKernelGGL(act_quant_kernel<0>, dim3((unsigned)blocks), dim3(AQ_THREADS), 0, stream,
                           reinterpret_cast<const u32x4 *>(x), reinterpret_cast<u32x2 *>(q), s, n_tiles, by_nkb, M);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// weight_quant: one workgroup (256 threads) per 128x128 block. Thread t covers the
// 16-byte chunk (t & 15) of rows (t >> 4) + 16 i, i = 0..7. Rows past N (ragged last
// block row) are neither read nor written and do not enter the block's amax.
// ------------------------------------------------------------------------------------
constexpr int WQ_THREADS = 256;

__global__ __launch_bounds__(WQ_THREADS) void weight_quant_kernel(const uint16_t *__restrict__ w,
                                                                  uint8_t *__restrict__ q,
                                                                  float *__restrict__ s,
                                                                  int64_t N, int64_t K) {
    __shared__ uint32_t wave_max[WQ_THREADS / 64];
    const int64_t kb = blockIdx.x, nb = blockIdx.y;
    const int64_t nkb = K / kBlock;
    const int t = threadIdx.x;
    const int chunk = t & 15;
    const int64_t row0 = nb * kBlock + (t >> 4);

    u32x4 v[8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t r = row0 + 16 * i;
        v[i] = (r < N) ? *reinterpret_cast<const u32x4 *>(w + r * K + kb * kBlock + chunk * 8)
                       : u32x4{0, 0, 0, 0};
        uint32_t a = absmax_bits8(v[i]);
        m = m > a ? m : a;
    }
    m = row16_max(m);
    // combine the four DPP rows of the wave, then the four waves
    uint32_t r0 = __builtin_amdgcn_readlane(m, 0), r1 = __builtin_amdgcn_readlane(m, 16);
    uint32_t r2 = __builtin_amdgcn_readlane(m, 32), r3 = __builtin_amdgcn_readlane(m, 48);
    r0 = r0 > r1 ? r0 : r1;
    r2 = r2 > r3 ? r2 : r3;
    if ((t & 63) == 0) wave_max[t >> 6] = r0 > r2 ? r0 : r2;
    __syncthreads();
    uint32_t amax = wave_max[0];
#pragma unroll
    for (int i = 1; i < WQ_THREADS / 64; ++i) amax = amax > wave_max[i] ? amax : wave_max[i];

    TileScale ts = tile_scale(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t r = row0 + 16 * i;
        u32x2 codes = quant8(v[i], ts);
        if (r < N) *reinterpret_cast<u32x2 *>(q + r * K + kb * kBlock + chunk * 8) = codes;
    }
    if (t == 0) s[nb * nkb + kb] = ts.s;
}

hipError_t launch_weight_quant(const uint16_t *w, uint8_t *q, float *s, int64_t N, int64_t K,
                               hipStream_t stream) {
    const int64_t nkb = K / kBlock, nnb = (N + kBlock - 1) / kBlock;
    if (nkb == 0 || nnb == 0) return hipSuccess;
    hipLaunchKernelGGL(weight_quant_kernel, dim3((unsigned)nkb, (unsigned)nnb), dim3(WQ_THREADS), 0,
                       stream, w, q, s, N, K);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// weight_dequant: each thread turns 16-byte chunks of codes (16 consecutive k inside one
// 128-wide block) into 16 bf16 values: decode (v_cvt_pk_f32_fp8), one fp32 multiply by the
// block scale, round to bf16 (v_cvt_pk_bf16_f32). Grid-stride over the chunks, so the
// launch stays within the 32-bit work-item count of a grid dimension at any size.
// ------------------------------------------------------------------------------------
constexpr int DQ_THREADS = 256;

template <bool HI>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t word, float sc) {
    f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
    return pack_bf16x2(f[0] * sc, f[1] * sc);
}

__global__ __launch_bounds__(DQ_THREADS) void weight_dequant_kernel(const u32x4 *__restrict__ q,
                                                                    const float *__restrict__ s,
                                                                    u32x4 *__restrict__ w,
                                                                    int64_t n_chunks, int64_t K) {
    const int64_t chunks_per_row = K / 16;
    for (int64_t c = (int64_t)blockIdx.x * DQ_THREADS + threadIdx.x; c < n_chunks;
         c += (int64_t)gridDim.x * DQ_THREADS) {
        const int64_t n = c / chunks_per_row;
        const int64_t k = (c - n * chunks_per_row) * 16;
        const float sc = s[(n / kBlock) * (K / kBlock) + k / kBlock];
        const u32x4 v = __builtin_nontemporal_load(&q[c]);
        u32x4 o0, o1;
        o0.x = dequant_pair<false>(v.x, sc);
        o0.y = dequant_pair<true>(v.x, sc);
        o0.z = dequant_pair<false>(v.y, sc);
        o0.w = dequant_pair<true>(v.y, sc);
        o1.x = dequant_pair<false>(v.z, sc);
        o1.y = dequant_pair<true>(v.z, sc);
        o1.z = dequant_pair<false>(v.w, sc);
        o1.w = dequant_pair<true>(v.w, sc);
        // ordinary stores: the bf16 weight stays in the MALL for the GEMM that reads it next
        // (the bf16 branch of linear(); measured on the q down-projection's weight: the GEMM
        // after the dequant 127 -> 96 us with the dequant itself 10.5 -> 11.4 us)
        w[2 * c] = o0;
        w[2 * c + 1] = o1;
    }
}

hipError_t launch_weight_dequant(const uint8_t *q, const float *s, uint16_t *w, int64_t N, int64_t K,
                                 hipStream_t stream) {
    const int64_t n_chunks = N * (K / 16);
    if (n_chunks == 0) return hipSuccess;
    // 64 workgroups per CU, then grid-stride (an offline kernel: the loop costs nothing measurable)
    const int64_t cap = (int64_t)256 * 64;
    const int64_t want = (n_chunks + DQ_THREADS - 1) / DQ_THREADS;
    const int64_t blocks = want < cap ? want : cap;
    hipLaunchKernelGGL(weight_dequant_kernel, dim3((unsigned)blocks), dim3(DQ_THREADS), 0, stream,
                       reinterpret_cast<const u32x4 *>(q), s, reinterpret_cast<u32x4 *>(w), n_chunks, K);
    return hipGetLastError();
}

}  // namespace fp8q
