// bf16_gemm.hip -- Y = X . W^T on bf16 operands for gfx950: the bf16 branch of linear().
//
// What it computes (pomoai.com "DeepSeek-V3", section "FP8 mixed-precision training", the
// linear() listing: when the GEMM is not done in FP8, the FP8 weight is first dequantised
// to bf16 by weight_dequant and the layer is a plain bf16 linear, y = x . W^T (+ bias)):
//     Y[m, n] = sum_k X[m, k] * W[n, k]   (+ bias[n])
// with every product exact in fp32 (bf16 x bf16) and the sum accumulated in fp32 by the
// matrix unit; the output is fp32 or RN_bf16 of the fp32 accumulator.
//
// Contraction. v_mfma_f32_16x16x32_bf16 with the accumulator chained across K, so there is
// no per-slice promotion here (there are no scales). As in the block GEMM, W rows are the
// MFMA's A operand and X rows its B operand: lane l of a 16x16 result holds n = 4*(l/16) + r
// (r = 0..3) for m = l % 16, four consecutive outputs of a row of Y.
//
// Tiling. A workgroup of 8 waves owns a 256 x 128 output tile; its waves form a 4 x 2 grid
// of 64 x 64 wave tiles (4 x 4 blocks of 16 x 16). K advances in steps of 64 elements, one
// 128-byte piece of every tile row, copied global -> LDS by LDS-DMA loads (buffer_load ...
// lds) into one of 3 stage buffers; 16-byte chunks of each row are XOR-swizzled by (row & 7)
// so that the fragment reads (16 rows x 4 chunks per instruction) are free of bank
// conflicts. Rows past M or N lie outside the loads' buffer range and read as zero.
//
// Work order. Workgroups are dealt round-robin to the 8 XCDs; the block index is remapped
// so that each XCD walks a contiguous run of tiles, taken down `group` tile rows per tile
// column, so that the tiles one XCD holds at once share A and W panels in its L2.
#include "device_common.h"
#include "launch.h"

namespace fp8q {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int BM = 256, BN = 128, NW = 8, WAVES_M = 4, WAVES_N = 2;
constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;       // 64 x 64 per wave
constexpr int SUB_M = WM / 16, SUB_N = WN / 16;           // 4 x 4 blocks
constexpr int KSTEP = 64;                                 // bf16 elements per stage row
constexpr int ROW_BYTES = KSTEP * 2;                      // 128
constexpr int NSTAGE = 3;
constexpr int A_BYTES = BM * ROW_BYTES, W_BYTES = BN * ROW_BYTES;
constexpr int STAGE = A_BYTES + W_BYTES;                  // 48 KiB
constexpr int A_INSTR = BM / (8 * NW), W_INSTR = BN / (8 * NW);   // 1 KiB copies per wave and stage
constexpr int IPW = A_INSTR + W_INSTR;
static_assert(STAGE * NSTAGE <= 160 * 1024, "LDS budget");

struct Bf16GemmArgs {
    const uint16_t *x;
    const uint16_t *w;
    const float *bias;   // [N] or null
    void *y;
    int64_t M, N, K;
    int tiles_m, tiles_n, group;
};

__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ rsrc_t make_rsrc(const void *p, int64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// two 16x16x32 bf16 MFMAs over one 64-wide K step: the fragment's first 16 bytes hold this
// lane's k = 8g .. 8g+7, its second 16 bytes k = 32 + 8g .. 32 + 8g + 7 (g = lane / 16),
// the same in both operands
__device__ __forceinline__ f32x4 mfma_step(const u32x4 (&w)[2], const u32x4 (&x)[2], f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[0]), __builtin_bit_cast(bf16x8, x[0]),
                                                  acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[1]), __builtin_bit_cast(bf16x8, x[1]),
                                                   acc, 0, 0, 0);
}

template <int OUT_BF16>
__global__ __launch_bounds__(NW * 64) void bf16_gemm_kernel(Bf16GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[STAGE * NSTAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;

    // XCD-contiguous logical tile index (workgroup b runs on XCD b % 8), then down `group`
    // tile rows per tile column
    const int tiles = g.tiles_m * g.tiles_n;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int q = tiles >> 3, rem = tiles & 7;
    const int tl = xcd * q + (xcd < rem ? xcd : rem) + slot;
    const int band = tl / (g.group * g.tiles_n);
    const int in_band = tl - band * g.group * g.tiles_n;
    const int band_rows = min(g.group, g.tiles_m - band * g.group);
    const int64_t m0 = (int64_t)(band * g.group + in_band % band_rows) * BM;
    const int64_t n0 = (int64_t)(in_band / band_rows) * BN;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int64_t row_bytes = K * 2;
    const int nks = (int)(K / KSTEP);

    // copies: instruction t of wave w moves tile rows 8 (NW t + w) .. + 7; lane L fills
    // LDS row L / 8, physical chunk L % 8, i.e. loads the logical chunk swz_chunk maps there
    const rsrc_t rx = make_rsrc(g.x + m0 * K, (M - m0 < BM ? M - m0 : BM) * row_bytes);
    const rsrc_t rw = make_rsrc(g.w + n0 * K, (N - n0 < BN ? N - n0 : BN) * row_bytes);
    uint32_t off[IPW];
    const int sub = lane >> 3;
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
        const int tt = t < A_INSTR ? t : t - A_INSTR;
        const int row = 8 * (NW * tt + wave) + sub;
        off[t] = (uint32_t)(row * row_bytes) + (swz_chunk(row, lane & 7) << 4);
    }
    auto issue = [&](int ks, int st) __device__ __attribute__((always_inline)) {
        const int koff = __builtin_amdgcn_readfirstlane(ks * ROW_BYTES);
        uint8_t *base = smem + st * STAGE;
#pragma unroll
        for (int t = 0; t < IPW; ++t) {
            if (t < A_INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(base + 8 * (NW * t + wave) * ROW_BYTES), 16,
                                                         off[t], koff, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (lds_void *)(base + A_BYTES + 8 * (NW * (t - A_INSTR) + wave) * ROW_BYTES), 16, off[t], koff,
                    0, 0);
        }
    };

    f32x4 acc[SUB_M][SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment read offsets within a stage: row frow of a 16-row group, logical chunks g
    // and 4 + g
    const int frow = lane & 15, kg = lane >> 4;
    const int lo = frow * ROW_BYTES + (swz_chunk(frow, kg) << 4);
    const int hi = frow * ROW_BYTES + (swz_chunk(frow, 4 + kg) << 4);
    const int a_base = wm * WM * ROW_BYTES, w_base = A_BYTES + wn * WN * ROW_BYTES;
    auto frag = [&](const uint8_t *p, u32x4 (&f)[2]) __device__ __attribute__((always_inline)) {
        f[0] = *reinterpret_cast<const u32x4 *>(p + lo);
        f[1] = *reinterpret_cast<const u32x4 *>(p + hi);
    };

    // prologue: the first NSTAGE - 1 steps in flight
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nks) issue(s, s);

    for (int ks = 0; ks < nks; ++ks) {
        const int st = ks % NSTAGE;
        // step ks has landed once at most the copies of the steps queued after it are in
        // flight (loads retire in issue order); then every wave's copies are visible after
        // the barrier, which also means every wave is done reading step ks - 1
        if (ks + 1 < nks) wait_vmcnt<IPW * (NSTAGE - 2)>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (ks + NSTAGE - 1 < nks) issue(ks + NSTAGE - 1, (ks + NSTAGE - 1) % NSTAGE);
        const uint8_t *stage = smem + st * STAGE;
        u32x4 wf[SUB_N][2], xf[2], xn[2];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) frag(stage + w_base + 16 * j * ROW_BYTES, wf[j]);
        frag(stage + a_base, xf);
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) {
            if (i + 1 < SUB_M) frag(stage + a_base + 16 * (i + 1) * ROW_BYTES, xn);
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) acc[i][j] = mfma_step(wf[j], xf, acc[i][j]);
            if (i + 1 < SUB_M) {
                xf[0] = xn[0];
                xf[1] = xn[1];
            }
        }
    }

    // epilogue: bias (fp32) added before the output rounding; stores masked to [M, N)
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) {
        const int64_t n = n0 + wn * WN + 16 * j + 4 * kg;
        f32x4 b = {0.f, 0.f, 0.f, 0.f};
        if (g.bias) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) b[r] = g.bias[n + r];
        }
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) {
            const int64_t m = m0 + wm * WM + 16 * i + frow;
            if (m >= M || n >= N) continue;
            const f32x4 v = acc[i][j] + b;
            if constexpr (OUT_BF16) {
                uint16_t *yp = reinterpret_cast<uint16_t *>(g.y) + m * N + n;
                if (n + 4 <= N && (((uintptr_t)yp) & 7) == 0) {
                    *reinterpret_cast<u32x2 *>(yp) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) yp[r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xFFFF);
                }
            } else {
                float *yp = reinterpret_cast<float *>(g.y) + m * N + n;
                if (n + 4 <= N && (((uintptr_t)yp) & 15) == 0) {
                    *reinterpret_cast<f32x4 *>(yp) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) yp[r] = v[r];
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_bf16_gemm(const uint16_t *x, const uint16_t *w, const float *bias, void *y, bool out_bf16, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    Bf16GemmArgs a{x, w, bias, y, M, N, K, (int)((M + BM - 1) / BM), (int)((N + BN - 1) / BN), 1};
    // group: tile rows walked per tile column, so that an XCD's ~32 resident tiles form a
    // compact block (fewest A + W rows); as in the block GEMM's planner
    int64_t best_rows = -1;
    for (int gsz = 1; gsz <= 32; gsz *= 2) {
        const int64_t gg = gsz < a.tiles_m ? gsz : a.tiles_m;
        const int64_t cols = (32 + gg - 1) / gg;
        const int64_t rows = gg * BM + (cols < a.tiles_n ? cols : a.tiles_n) * BN;
        if (best_rows < 0 || rows < best_rows) {
            best_rows = rows;
            a.group = gsz;
        }
    }
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles * NW * 64 > 0xFFFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles), block(NW * 64);
    // (K = 0 runs no K step: Y is the bias, or zero)
    if (out_bf16)
        bf16_gemm_kernel<1><<<grid, block, 0, stream>>>(a);
    else
        bf16_gemm_kernel<0><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace fp8q
