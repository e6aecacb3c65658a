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
// Tiling. Three tiles: 256 x 256 with 8 waves of 128 x 64 (8 x 4 blocks of 16 x 16) for
// large shapes with long K; 128 x 128 with 4 waves of 64 x 64 (two workgroups per CU); and
// 64 x 128 with 4 waves of 32 x 64 for shapes with too few 128 x 128 tiles. K advances in
// steps of 64 elements, one 128-byte piece of every tile row, copied global -> LDS by LDS-DMA
// loads (buffer_load ... lds) into one of NSTAGE stage buffers; 16-byte chunks of each row
// are XOR-swizzled by (row & 7) so that the fragment reads (16 rows x 4 chunks per
// instruction) are free of bank conflicts. Rows past M or N lie outside the loads' buffer
// range and read as zero.
//
// Schedule. 32 x 64 and 64 x 64 wave tiles: two register sets hold the fragments of two K
// steps; the MFMAs of step ks take their operands from one set while the other is filled
// from LDS with step ks + 1, so the LDS reads have a whole step of MFMA work to land behind,
// and a stage buffer is free once its step is in registers (the copies of step ks + NSTAGE
// go into the buffer of step ks). 128 x 64 wave tiles (two such sets do not fit beside 128
// accumulator registers): the step's W fragments are read first and its A fragments one row
// group ahead of their MFMAs. Per step a 128 x 64 wave reads 24 KB of fragments for 1024
// cycles of MFMA work, a 64 x 64 one 16 KB for 512, which is why the larger tile leads
// where it fills the GPU and K is long.
//
// Epilogue. The output goes through LDS and leaves in 16-byte stores that write whole
// 128-byte pieces of output rows.
//
// Work order. Workgroups are dealt round-robin to the 8 XCDs; the block index is remapped
// so that each XCD walks a contiguous run of tiles, taken down `group` tile rows per tile
// column, so that the tiles one XCD holds at once share A and W panels in its L2.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "launch.h"

namespace fp8q {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int KSTEP = 64;                                 // bf16 elements per stage row
constexpr int ROW_BYTES = KSTEP * 2;                      // 128

// tile configuration: BM x BN, NW waves in a WAVES_M x (NW / WAVES_M) grid, NSTAGE stages
template <int BM_, int BN_, int NW_, int WAVES_M_, int NSTAGE_>
struct Bf16Tile {
    static constexpr int BM = BM_, BN = BN_, NW = NW_, WAVES_M = WAVES_M_, WAVES_N = NW_ / WAVES_M_;
    static constexpr int NSTAGE = NSTAGE_;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;      // wave tile
    static constexpr int SUB_M = WM / 16, SUB_N = WN / 16;
    static constexpr int A_BYTES = BM * ROW_BYTES, W_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE = A_BYTES + W_BYTES;
    static constexpr int A_INSTR = BM / (8 * NW), W_INSTR = BN / (8 * NW);   // 1 KiB copies per wave and stage
    static constexpr int IPW = A_INSTR + W_INSTR;
    // register prefetch of whole steps where two sets of a step's fragments fit (wave tiles
    // of 32 x 64 and 64 x 64); the 128 x 64 wave tile streams its A fragments through the
    // step instead
    static constexpr bool PF = WM <= 64;
    static_assert(WAVES_M * WAVES_N == NW && WN == 64 && (WM == 32 || WM == 64 || WM == 128), "wave tiles");
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "copy rows");
    static_assert(STAGE * NSTAGE <= 160 * 1024, "LDS budget");
    static_assert(NSTAGE >= 2 && IPW * (NSTAGE - 1) < 64, "stages");
};
using TileXL = Bf16Tile<256, 256, 8, 2, 2>;   // 256 x 256, 8 waves of 128 x 64, 128 KiB of LDS
using TileS = Bf16Tile<128, 128, 4, 2, 2>;    // 128 x 128, 4 waves, 64 KiB (two workgroups per CU)
using TileM = Bf16Tile<64, 128, 4, 2, 2>;     // 64 x 128, 4 waves of 32 x 64, 48 KiB

// Output staging of the epilogue: rounds of IPR row groups (RG = 16 x WAVES_M tile rows
// each) in LDS rows of LDS_ROW bytes, padded so that both the fragment writes and the row
// reads are free of bank conflicts. BYTES is the LDS the kernel needs for it: the stage
// buffers, or the whole tile in one round where that fits beside the kernel's occupancy.
template <class T, int OUT_BF16>
struct Bf16Epilogue {
    static constexpr int OB = OUT_BF16 ? 2 : 4;                 // bytes per output element
    static constexpr int EPC = 16 / OB;                         // elements per 16-byte chunk
    static constexpr int ROW_WORDS = T::BN * OB / 4;
    static constexpr int TARGET = OUT_BF16 ? 8 : 16;            // row stride, in banks, mod 64
    static constexpr int LDS_ROW = 4 * (ROW_WORDS + ((TARGET - ROW_WORDS) % 64 + 64) % 64);
    static constexpr int RG = T::WAVES_M * 16;
    static constexpr int CPR = T::BN * OB / 16;                 // 16-byte chunks per output row
    static constexpr int STAGES = T::STAGE * T::NSTAGE;
    static constexpr int ALL = T::SUB_M * RG * LDS_ROW;         // the whole tile at once
    // (the 4-wave tiles run two or more workgroups per CU: their LDS stays within 80 KB)
    static constexpr int LIMIT = T::NW == 8 ? 160 * 1024 : 80 * 1024;
    static constexpr bool ONE_ROUND = ALL <= (STAGES > LIMIT ? STAGES : LIMIT);
    static constexpr int BYTES = ONE_ROUND && ALL > STAGES ? ALL : STAGES;
    static constexpr int IPR0 = STAGES / (RG * LDS_ROW);
    static constexpr int IPR = ONE_ROUND ? T::SUB_M : (IPR0 < T::SUB_M ? IPR0 : T::SUB_M);
    static_assert(IPR >= 1, "epilogue staging does not fit");
};

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

// This wave's LDS-DMA copies. Instruction t of wave w moves tile rows 8 (NW t + w) .. + 7
// of X (t < A_INSTR), then of W; lane L fills LDS row L / 8 of those 8, physical chunk L % 8,
// i.e. loads the logical chunk that swz_chunk maps there. OUT_BF16 makes the type unique to
// each kernel instantiation (the host pass emits a launch stub for only one kernel among
// those that share such a type, and the resource type may appear in no signature it sees).
template <class T, int OUT_BF16>
struct Bf16Dma {
    rsrc_t rx, rw;
    uint32_t off[T::IPW];
    int wave;
    uint8_t *smem;

    __device__ __forceinline__ Bf16Dma(const uint16_t *x, const uint16_t *w, int64_t m0, int64_t n0, int64_t M,
                                       int64_t N, int64_t K, int wave_, int lane, uint8_t *smem_)
        : wave(wave_), smem(smem_) {
        const int64_t row_bytes = K * 2;
        rx = make_rsrc(x + m0 * K, (M - m0 < T::BM ? M - m0 : T::BM) * row_bytes);
        rw = make_rsrc(w + n0 * K, (N - n0 < T::BN ? N - n0 : T::BN) * row_bytes);
        const int sub = lane >> 3;
#pragma unroll
        for (int t = 0; t < T::IPW; ++t) {
            const int tt = t < T::A_INSTR ? t : t - T::A_INSTR;
            const int row = 8 * (T::NW * tt + wave) + sub;
            off[t] = (uint32_t)(row * row_bytes) + (swz_chunk(row, lane & 7) << 4);
        }
    }

    // the copies of K step ks into its stage buffer
    __device__ __forceinline__ void issue(int ks) const {
        uint8_t *base = smem + (ks % T::NSTAGE) * T::STAGE;
        const int koff = __builtin_amdgcn_readfirstlane(ks * ROW_BYTES);
#pragma unroll
        for (int t = 0; t < T::IPW; ++t) {
            if (t < T::A_INSTR)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(base + 8 * (T::NW * t + wave) * ROW_BYTES),
                                                         16, off[t], koff, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (lds_void *)(base + T::A_BYTES + 8 * (T::NW * (t - T::A_INSTR) + wave) * ROW_BYTES), 16,
                    off[t], koff, 0, 0);
        }
    }
};

// this wave's fragments of K step ks: W column groups, then X row groups
template <class T>
__device__ __forceinline__ void read_step(const uint8_t *smem, int ks, int a_base, int w_base, int lo, int hi,
                                          u32x4 (&wf)[T::SUB_N][2], u32x4 (&xf)[T::SUB_M][2]) {
    const uint8_t *stage = smem + (ks % T::NSTAGE) * T::STAGE;
#pragma unroll
    for (int j = 0; j < T::SUB_N; ++j) {
        wf[j][0] = *reinterpret_cast<const u32x4 *>(stage + w_base + 16 * j * ROW_BYTES + lo);
        wf[j][1] = *reinterpret_cast<const u32x4 *>(stage + w_base + 16 * j * ROW_BYTES + hi);
    }
#pragma unroll
    for (int i = 0; i < T::SUB_M; ++i) {
        xf[i][0] = *reinterpret_cast<const u32x4 *>(stage + a_base + 16 * i * ROW_BYTES + lo);
        xf[i][1] = *reinterpret_cast<const u32x4 *>(stage + a_base + 16 * i * ROW_BYTES + hi);
    }
}

template <class T>
__device__ __forceinline__ void wait_step_landed(int queued_after) {
    // loads retire in issue order: a step has landed once at most the copies of the
    // `queued_after` steps issued after it are in flight
    if constexpr (T::NSTAGE >= 3) {
        if (queued_after >= 1) {
            wait_vmcnt<T::IPW * (T::NSTAGE - 2)>();
            return;
        }
    }
    wait_vmcnt<0>();
}

// K step ks, whose fragments are in (wf, xf): once every wave has them in registers (the
// barrier) its stage buffer takes step ks + NSTAGE; step ks + 1, visible after the same
// barrier, is read into (wf_next, xf_next) while the MFMAs of step ks run
template <class T, class Dma>
__device__ __forceinline__ void k_step(int ks, int nks, const Dma &dma, const uint8_t *smem, int a_base, int w_base,
                                       int lo, int hi,
                                       const u32x4 (&wf)[T::SUB_N][2], const u32x4 (&xf)[T::SUB_M][2],
                                       u32x4 (&wf_next)[T::SUB_N][2], u32x4 (&xf_next)[T::SUB_M][2],
                                       f32x4 (&acc)[T::SUB_M][T::SUB_N]) {
    const bool more = ks + 1 < nks;
    __builtin_amdgcn_sched_barrier(0);   // the waits stay behind the previous step's MFMAs
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0): (wf, xf) have landed
    if (more) wait_step_landed<T>(min(nks - 2 - ks, T::NSTAGE - 2));
    lds_barrier();
    if (ks + T::NSTAGE < nks) dma.issue(ks + T::NSTAGE);
    if (more) read_step<T>(smem, ks + 1, a_base, w_base, lo, hi, wf_next, xf_next);
#pragma unroll
    for (int i = 0; i < T::SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < T::SUB_N; ++j) acc[i][j] = mfma_step(wf[j], xf[i], acc[i][j]);
}

// All K steps with the A fragments streamed (the 128 x 64 wave tile, two stages). Per step:
// the W fragments are read first, then row group by row group the next group's A fragment is
// read while the current group's MFMAs run; at the end of the step every wave has read the
// step (the lgkmcnt wait) and waited for the next step's copies, and after the barrier the
// freed buffer takes the copies of step ks + 2, one step of lead.
template <class T, class Dma>
__device__ __forceinline__ void stream_steps(int nks, const Dma &dma, const uint8_t *smem, int a_base, int w_base,
                                             int lo, int hi, f32x4 (&acc)[T::SUB_M][T::SUB_N]) {
    static_assert(T::NSTAGE == 2, "two stages");
    dma.issue(0);
    if (nks > 1) dma.issue(1);
    if (nks > 1) wait_vmcnt<T::IPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    for (int ks = 0; ks < nks; ++ks) {
        const uint8_t *stage = smem + (ks & 1) * T::STAGE;
        u32x4 wf[T::SUB_N][2];
#pragma unroll
        for (int j = 0; j < T::SUB_N; ++j) {
            wf[j][0] = *reinterpret_cast<const u32x4 *>(stage + w_base + 16 * j * ROW_BYTES + lo);
            wf[j][1] = *reinterpret_cast<const u32x4 *>(stage + w_base + 16 * j * ROW_BYTES + hi);
        }
        u32x4 xa[2] = {*reinterpret_cast<const u32x4 *>(stage + a_base + lo),
                       *reinterpret_cast<const u32x4 *>(stage + a_base + hi)};
#pragma unroll
        for (int i = 0; i < T::SUB_M; ++i) {
            u32x4 xn[2] = {xa[0], xa[1]};
            if (i + 1 < T::SUB_M) {
                xn[0] = *reinterpret_cast<const u32x4 *>(stage + a_base + 16 * (i + 1) * ROW_BYTES + lo);
                xn[1] = *reinterpret_cast<const u32x4 *>(stage + a_base + 16 * (i + 1) * ROW_BYTES + hi);
            }
#pragma unroll
            for (int j = 0; j < T::SUB_N; ++j) acc[i][j] = mfma_step(wf[j], xa, acc[i][j]);
            xa[0] = xn[0];
            xa[1] = xn[1];
        }
        __builtin_amdgcn_sched_barrier(0);   // the waits stay behind this step's MFMAs
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
        if (ks + 1 < nks) wait_vmcnt<0>();   // step ks + 1 has landed
        lds_barrier();
        if (ks + 2 < nks) dma.issue(ks + 2);
    }
}

template <int BM_, int BN_, int NW_, int WAVES_M_, int NSTAGE_, int OUT_BF16>
__global__ __launch_bounds__(NW_ * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void bf16_gemm_kernel(
    Bf16GemmArgs g) {   // (2 waves per SIMD: the 4-wave tile runs two workgroups per CU)
    using T = Bf16Tile<BM_, BN_, NW_, WAVES_M_, NSTAGE_>;
    constexpr int NW = T::NW, WAVES_M = T::WAVES_M, WM = T::WM, WN = T::WN, SUB_M = T::SUB_M, SUB_N = T::SUB_N;
    constexpr int BM = T::BM, BN = T::BN, NSTAGE = T::NSTAGE, IPW = T::IPW;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Bf16Epilogue<T, OUT_BF16>::BYTES];

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
    const int nks = (int)(K / KSTEP);
    const Bf16Dma<T, OUT_BF16> dma(g.x, g.w, m0, n0, M, N, K, wave, lane, smem);

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
    const int a_base = wm * WM * ROW_BYTES, w_base = T::A_BYTES + wn * WN * ROW_BYTES;

    if constexpr (!T::PF) {
        if (nks > 0) stream_steps<T>(nks, dma, smem, a_base, w_base, lo, hi, acc);
    } else if (nks > 0) {
        // two register sets of fragments; step ks uses set ks % 2
        u32x4 wf0[SUB_N][2], xf0[SUB_M][2], wf1[SUB_N][2], xf1[SUB_M][2];
        // prologue: the first NSTAGE steps in flight, step 0 read into set 0
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s)
            if (s < nks) dma.issue(s);
        if (nks >= NSTAGE) wait_vmcnt<IPW * (NSTAGE - 1)>();
        else wait_vmcnt<0>();
        lds_barrier();
        read_step<T>(smem, 0, a_base, w_base, lo, hi, wf0, xf0);
        for (int ks = 0; ks < nks; ks += 2) {
            k_step<T>(ks, nks, dma, smem, a_base, w_base, lo, hi, wf0, xf0, wf1, xf1, acc);
            if (ks + 1 < nks) k_step<T>(ks + 1, nks, dma, smem, a_base, w_base, lo, hi, wf1, xf1, wf0, xf0, acc);
        }
    }

    // Epilogue, staged through LDS (every wave is past its last fragment read at the first
    // barrier): IPR row groups of every wave per round are written to LDS as output rows (bias
    // added in fp32 before the output rounding), then the workgroup stores them 16 bytes per
    // lane, so that each store instruction writes whole 128-byte pieces of output rows
    // (stored straight from the fragments, each line would be written in 8- or 16-byte pieces
    // by four instructions, which costs far more on output-heavy shapes). Stores are masked
    // to [M, N).
    {
        using E = Bf16Epilogue<T, OUT_BF16>;
        constexpr int OB = E::OB, EPC = E::EPC, LDS_ROW = E::LDS_ROW, RG = E::RG, IPR = E::IPR, CPR = E::CPR;
        constexpr int NT = NW * 64;
        // every output row 16-byte aligned (the interface asks only 4-byte alignment of y)
        const bool vec_ok = ((N * OB) & 15) == 0 && (reinterpret_cast<uintptr_t>(g.y) & 15) == 0;
        f32x4 bvec[SUB_N];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
            bvec[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (g.bias) {
                const int64_t n = n0 + wn * WN + 16 * j + 4 * kg;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) bvec[j][r] = g.bias[n + r];
            }
        }
#pragma unroll
        for (int i0 = 0; i0 < SUB_M; i0 += IPR) {
            __syncthreads();
#pragma unroll
            for (int ii = 0; ii < IPR; ++ii) {
                if (i0 + ii < SUB_M) {
                    uint8_t *rowp = smem + (ii * RG + wm * 16 + frow) * LDS_ROW;
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) {
                        const int col = wn * WN + 16 * j + 4 * kg;
                        const f32x4 v = acc[i0 + ii][j] + bvec[j];
                        if constexpr (OUT_BF16)
                            *reinterpret_cast<u32x2 *>(rowp + col * 2) =
                                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        else
                            *reinterpret_cast<f32x4 *>(rowp + col * 4) = v;
                    }
                }
            }
            __syncthreads();
            const int groups = (SUB_M - i0) < IPR ? (SUB_M - i0) : IPR;   // a constant once unrolled
            const int chunks = groups * RG * CPR;
            for (int c = threadIdx.x; c < chunks; c += NT) {
                const int r = c / CPR, cb = c - r * CPR;
                const int ii = r / RG, within = r - ii * RG;
                const int64_t m = m0 + (within >> 4) * WM + 16 * (i0 + ii) + (within & 15);
                const int64_t n = n0 + cb * EPC;
                if (m >= M || n >= N) continue;
                const uint8_t *src = smem + r * LDS_ROW + cb * 16;
                uint8_t *yp = reinterpret_cast<uint8_t *>(g.y) + (m * N + n) * OB;
                if (vec_ok && n + EPC <= N) {
                    *reinterpret_cast<u32x4 *>(yp) = *reinterpret_cast<const u32x4 *>(src);
                } else {
                    for (int e = 0; e < EPC && n + e < N; ++e) {
                        if constexpr (OUT_BF16)
                            reinterpret_cast<uint16_t *>(yp)[e] = reinterpret_cast<const uint16_t *>(src)[e];
                        else
                            reinterpret_cast<float *>(yp)[e] = reinterpret_cast<const float *>(src)[e];
                    }
                }
            }
        }
    }
}

}  // namespace

namespace {

template <class T>
hipError_t launch_tile(Bf16GemmArgs a, bool out_bf16, hipStream_t stream) {
    a.tiles_m = (int)((a.M + T::BM - 1) / T::BM);
    a.tiles_n = (int)((a.N + T::BN - 1) / T::BN);
    // group: tile rows walked per tile column, so that an XCD's ~32 resident tiles form a
    // compact block (fewest A + W rows)
    int64_t best_rows = -1;
    for (int gsz = 1; gsz <= 32; gsz *= 2) {
        const int64_t gg = gsz < a.tiles_m ? gsz : a.tiles_m;
        const int64_t cols = (32 + gg - 1) / gg;
        const int64_t rows = gg * T::BM + (cols < a.tiles_n ? cols : a.tiles_n) * T::BN;
        if (best_rows < 0 || rows < best_rows) {
            best_rows = rows;
            a.group = gsz;
        }
    }
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles * T::NW * 64 > 0xFFFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles), block(T::NW * 64);
    // (K = 0 runs no K step: Y is the bias, or zero)
    if (out_bf16)
        bf16_gemm_kernel<T::BM, T::BN, T::NW, T::WAVES_M, T::NSTAGE, 1><<<grid, block, 0, stream>>>(a);
    else
        bf16_gemm_kernel<T::BM, T::BN, T::NW, T::WAVES_M, T::NSTAGE, 0><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_gemm(const uint16_t *x, const uint16_t *w, const float *bias, void *y, bool out_bf16, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    Bf16GemmArgs a{x, w, bias, y, M, N, K, 0, 0, 1};
    // FP8Q_BF16_TILE=256x256, 128x128 or 64x128 forces a tile (tuning and tests). Otherwise
    // (measured on MI355X): 64x128 where 128x128 tiles would not give every CU more than one;
    // 256x256 where its tiles fill the 256 CUs and K is long enough (K >= 2048) for its
    // per-tile cost to pay off; else 128x128, two workgroups per CU.
    if (const char *e = std::getenv("FP8Q_BF16_TILE")) {
        if (std::strcmp(e, "256x256") == 0) return launch_tile<TileXL>(a, out_bf16, stream);
        if (std::strcmp(e, "128x128") == 0) return launch_tile<TileS>(a, out_bf16, stream);
        if (std::strcmp(e, "64x128") == 0) return launch_tile<TileM>(a, out_bf16, stream);
    }
    const int64_t s_tiles = ((M + TileS::BM - 1) / TileS::BM) * ((N + TileS::BN - 1) / TileS::BN);
    const int64_t xl_tiles = ((M + TileXL::BM - 1) / TileXL::BM) * ((N + TileXL::BN - 1) / TileXL::BN);
    if (s_tiles <= 256) return launch_tile<TileM>(a, out_bf16, stream);
    if (xl_tiles >= 256 && K >= 2048) return launch_tile<TileXL>(a, out_bf16, stream);
    return launch_tile<TileS>(a, out_bf16, stream);
}

}  // namespace fp8q
