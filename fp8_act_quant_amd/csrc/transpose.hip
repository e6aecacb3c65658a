// transpose.hip -- layout kernels for the FP8 training GEMMs (gfx950).
//
// Activation gradient:  dX = dY . W, a contraction over W's rows. The weight's 128x128 blocks
// are square, so the transposed weight has the same codes and block scales, only
// transposed: weight_transpose produces Wq^T and its scale grid once, and dX is an ordinary
// block-scaled GEMM of the quantised dY against them.
// Weight gradient:  dW = dY^T . X, a contraction over tokens. Both operands are quantised in
// 1x128 tiles along the token dimension (the activation rule of the forward pass applied to
// the contraction dimension) and written token-contiguous: act_quant_t.
//
// E4M3 is OCP E4M3FN; the scale and quotient rules are those of act_quant (device_common.h).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

// ------------------------------------------------------------------------------------
// act_quant_t: x [M, C] bf16 -> qt [C, ldq] codes, st [C, ldq / 128] scales,
// ldq = ceil(M / 128) * 128. One workgroup (256 threads) per 128 tokens x 128 channels.
// Thread t takes token group g = t % 16 (tokens 8g .. 8g+7 of the tile) and channel chunk
// q = t / 16 (channels 8q .. 8q+7): it loads 8 rows x 16 bytes, regroups them into eight
// 8-token vectors (one per channel), and the 16 lanes of a DPP row, which hold the 16 token
// groups of the same channels, reduce each channel's amax. Every lane then quantises its 8
// tokens of each channel and the 16 lanes write the channel's 128 codes as one 128-byte row
// piece. Tokens past M read as zero: they do not change an amax and encode to code 0.
// ------------------------------------------------------------------------------------
constexpr int AQT_THREADS = 256;

__global__ __launch_bounds__(AQT_THREADS) void act_quant_t_kernel(const uint16_t *__restrict__ x,
                                                                  uint8_t *__restrict__ qt,
                                                                  float *__restrict__ st, int64_t M,
                                                                  int64_t C, int64_t ldq) {
    const int t = threadIdx.x;
    const int g = t & 15, q = t >> 4;
    const int64_t mb = blockIdx.x;
    const int64_t c0 = (int64_t)blockIdx.y * 128 + q * 8;   // first channel of this lane
    const bool chunk_ok = c0 < C;                           // C is a multiple of 8
    const int64_t tok0 = mb * kBlock + g * 8;
    u32x4 row[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t m = tok0 + r;
        // (ordinary loads: a load instruction takes 64 bytes of each of 16 rows, and the
        // rest of each line, loaded by another wave, is then found in the L2; non-temporal
        // loads cost 27.0 against 20.2 us on a 4096 x 7168 input)
        row[r] = (chunk_ok && m < M) ? *reinterpret_cast<const u32x4 *>(x + m * C + c0)
                                     : u32x4{0, 0, 0, 0};
    }
    // col[e]: channel c0 + e over the 8 tokens, as 8 bf16 in token order (2 per word)
    u32x4 col[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        // selector for v_perm_b32(a, b, sel): bytes of b are 0..3, bytes of a are 4..7; the
        // low bf16 of a word is bytes 0-1, the high bf16 bytes 2-3
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint32_t v[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = row[2 * p][w], hi = row[2 * p + 1][w];
            v[p] = __builtin_amdgcn_perm(hi, lo, sel);   // token 2p in the low half, 2p+1 in the high half
        }
        col[e] = u32x4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t amax = row16_max(absmax_bits8(col[e]));
        const TileScale ts = tile_scale(amax);
        const u32x2 codes = quant8(col[e], ts);
        const int64_t c = c0 + e;
        if (chunk_ok) {
            *reinterpret_cast<u32x2 *>(qt + c * ldq + mb * kBlock + g * 8) = codes;
            if (g == 0) st[c * (ldq / kBlock) + mb] = ts.s;
        }
    }
}

hipError_t launch_act_quant_t(const uint16_t *x, uint8_t *qt, float *st, int64_t M, int64_t C, hipStream_t stream) {
    const int64_t nmb = (M + kBlock - 1) / kBlock, ncb = (C + 127) / 128;
    if (nmb == 0 || ncb == 0) return hipSuccess;
    hipLaunchKernelGGL(act_quant_t_kernel, dim3((unsigned)nmb, (unsigned)ncb), dim3(AQT_THREADS), 0, stream, x, qt,
                       st, M, C, nmb * kBlock);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// weight_transpose: codes [N, K] -> [K, N] through LDS, 64 x 64 bytes per workgroup
// (256 threads). Thread t loads 16 bytes of row t / 4, and after the barrier assembles
// 16 bytes of output row t / 4 (16 consecutive n of one k) from a column of the tile. The
// scale grid [ceil(N/128), K/128] -> [K/128, ceil(N/128)] is transposed by the workgroups of
// the first tile column, 256 entries per workgroup.
// ------------------------------------------------------------------------------------
constexpr int WT_THREADS = 256;
constexpr int WT_TILE = 64;
constexpr int WT_PITCH = WT_TILE + 4;   // LDS row pitch in bytes (column reads spread over banks)

__global__ __launch_bounds__(WT_THREADS) void weight_transpose_kernel(const uint8_t *__restrict__ wq,
                                                                      const float *__restrict__ sw,
                                                                      uint8_t *__restrict__ wqt,
                                                                      float *__restrict__ swt, int64_t N,
                                                                      int64_t K) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[WT_TILE * WT_PITCH];
    const int t = threadIdx.x;
    const int64_t k0 = (int64_t)blockIdx.x * WT_TILE, n0 = (int64_t)blockIdx.y * WT_TILE;
    {
        const int r = t >> 2, ch = t & 3;
        const int64_t n = n0 + r;
        u32x4 v = {0, 0, 0, 0};
        if (n < N) v = *reinterpret_cast<const u32x4 *>(wq + n * K + k0 + ch * 16);
        uint32_t *dst = reinterpret_cast<uint32_t *>(tile + r * WT_PITCH + ch * 16);
        dst[0] = v.x;
        dst[1] = v.y;
        dst[2] = v.z;
        dst[3] = v.w;
    }
    __syncthreads();
    {
        const int r = t >> 2, ch = t & 3;   // output row k0 + r, columns n0 + 16 ch .. +15
        uint32_t w[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) word |= (uint32_t)tile[(ch * 16 + 4 * b + i) * WT_PITCH + r] << (8 * i);
            w[b] = word;
        }
        const int64_t n = n0 + ch * 16;
        uint8_t *out = wqt + (k0 + r) * N + n;
        if (n + 16 <= N && (N & 15) == 0) {
            *reinterpret_cast<u32x4 *>(out) = u32x4{w[0], w[1], w[2], w[3]};
        } else {
            for (int i = 0; i < 16 && n + i < N; ++i) out[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        }
    }
    if (blockIdx.x == 0) {
        const int64_t nkb = K / kBlock, nnb = (N + kBlock - 1) / kBlock;
        for (int64_t e = (int64_t)blockIdx.y * WT_THREADS + t; e < nkb * nnb; e += (int64_t)gridDim.y * WT_THREADS) {
            const int64_t kb = e / nnb, nb = e - kb * nnb;
            swt[e] = sw[nb * nkb + kb];
        }
    }
}

hipError_t launch_weight_transpose(const uint8_t *wq, const float *sw, uint8_t *wqt, float *swt, int64_t N,
                                   int64_t K, hipStream_t stream) {
    const int64_t nkt = K / WT_TILE, nnt = (N + WT_TILE - 1) / WT_TILE;
    if (nkt == 0 || nnt == 0) return hipSuccess;
    hipLaunchKernelGGL(weight_transpose_kernel, dim3((unsigned)nkt, (unsigned)nnt), dim3(WT_THREADS), 0, stream, wq,
                       sw, wqt, swt, N, K);
    return hipGetLastError();
}

}  // namespace fp8q
