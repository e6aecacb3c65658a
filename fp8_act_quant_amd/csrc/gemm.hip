// gemm.hip -- block-scaled FP8 GEMM Y = A . W^T for gfx950.
//
// What it computes (qdgithub.com book 25/317, section "FP8 quantisation: balancing storage
// and compute": FP8 products inside each row/column block, dequantisation outside the
// matrix units; 88811315.cn post 75335: FP8 partials promoted into an FP32 main
// accumulator; pomoai.com "DeepSeek-V3", linear(): fp8_gemm(x, scale, weight,
// weight.scale), output not re-quantised):
//     Y[m, n] = sum_kb P[m, n, kb] * (sa[m, kb] * sw[n / 128, kb])
// with P the fp32 partial over the 128-wide K slice kb.
//
// Promotion. One v_mfma_f32_16x16x128_f8f6f4 contracts exactly one 128-wide slice of a
// 16x16 output block, so every MFMA starts from zero and its result is folded into the
// fp32 main accumulator with one FMA per element, scaled by that slice's sa * sw. (The
// matrix unit sums each group of 8 products at reduced alignment precision; only the
// per-slice result crosses into the fp32 accumulator, as the promotion scheme intends.)
//
// Orientation. The MFMA's A operand is a 16-row slice of W (rows n) and its B operand a
// 16-row slice of A (rows m): lane l of the 16x16 result holds n = 4*(l/16) + r (r = 0..3)
// for one m = l % 16, so a lane needs one activation scale per 16-row group of m and its
// four outputs are consecutive in a row of Y.
//
// Tiling. A 256-thread workgroup owns a BM x BN output tile; its 4 waves form a
// WAVES_M x WAVES_N grid, each owning (16*SUB_M) x (16*SUB_N). Both operands are
// K-contiguous. Each K slice of the tile (BM + BN rows of 128 bytes, plus the BM
// activation scales of that slice) is copied global -> LDS by the LDS-DMA loads
// (global_load_lds), bypassing registers, into one of NSTAGE buffers: the copies for
// slice kb + NSTAGE - 1 are in flight while slice kb is contracted. 16-byte chunks of a row
// are XOR-swizzled (swz_chunk) so that fragment reads are free of bank conflicts.
// Rows past M or N are clamped to the last valid row: they only feed outputs that are
// never stored.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int G_SLICE = 128;   // K slice = promotion interval = one f8f6f4 MFMA

template <int BM, int BN, int NSTAGE, int NW>
struct GemmSmem {
    static_assert(BM % 64 == 0 && BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile shape");
    static constexpr int A_BYTES = BM * G_SLICE;
    static constexpr int W_BYTES = BN * G_SLICE;
    static constexpr int SA_BYTES = BM * 4;
    static constexpr int SW_BYTES = 64 * 4;   // weight scales of the tile's N-blocks (<= 64)
    static constexpr int STAGE = A_BYTES + W_BYTES + SA_BYTES + SW_BYTES;
    static constexpr int TOTAL = STAGE * NSTAGE;
    // LDS-DMA instructions per wave and slice: each tile instruction moves 1 KiB (8 rows of
    // 128 B), each scale instruction 256 B (64 rows of one fp32)
    static constexpr int A_INSTR = BM / (8 * NW), W_INSTR = BN / (8 * NW), SA_INSTR = BM / 64;
    static constexpr int INSTR_PER_WAVE = A_INSTR + W_INSTR + 2;
};

// 16-byte chunk c of LDS row r is stored at physical chunk c ^ (r & 7). With the fragment
// reads below (one instruction: 16 rows x 4 consecutive logical chunks) every read is
// conflict-free on gfx950's LDS (measured: ~4 cycles per 1 KiB wave read).
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ (row & 7); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * G_SLICE + (swz_chunk(row, chunk) << 4); }

__device__ __forceinline__ f32x4 mfma_slice(const i32x8 &a, const i32x8 &b) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // format codes 0/0: both operands FP8 E4M3; scale operands 0 select the unscaled MFMA
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Exact-slice contraction. The FP8 matrix unit adds each group of 8 products after
// aligning them to the group's largest product with 13 fraction bits (measured), so a
// product more than ~2^7 below its group's largest loses low bits. For callers that need
// slice partials at fp32 accuracy, both fragments are converted exactly to f16 (every
// E4M3 value is a normal f16) and contracted by four 16x16x32 f16 MFMAs, whose products
// and sums are kept exactly within each instruction; the four are chained in fp32.
struct Frag16 {
    f16x8 q[4];   // q[i] holds the fragment's k values 8i .. 8i+7 (this lane's k order)
};

__device__ __forceinline__ Frag16 to_f16(const i32x8 &f) {
    Frag16 r;
#pragma unroll
    for (int d = 0; d < 8; d += 2) {
        const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f[d], 1.0f, false);
        const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f[d], 1.0f, true);
        const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f[d + 1], 1.0f, false);
        const f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f[d + 1], 1.0f, true);
        r.q[d / 2] = f16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
    }
    return r;
}

__device__ __forceinline__ f32x4 mfma_slice_exact(const Frag16 &a, const Frag16 &b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.q[q], b.q[q], acc, 0, 0, 0);
    return acc;
}

// fragment of one 16-row group: lane l supplies row (l % 16) and, with g = l / 16, the
// 16-byte chunks g and 4 + g of the 128-byte slice (k = 16g .. 16g+15 and 64+16g .. 64+16g+15).
// Both MFMA operands use this lane -> k mapping, so matching k are paired; each 8-byte half
// of a chunk is an aligned run of 8 consecutive k.
__device__ __forceinline__ i32x8 load_frag(const uint8_t *base, int row, int kgroup) {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + swz(row, kgroup));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + swz(row, 4 + kgroup));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt encoding on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Buffer resource over `bytes` bytes at p (raw buffer, 32-bit offsets). Loads at offsets
// >= bytes return zero instead of touching memory.
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, int64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}

// Per-lane LDS-DMA offsets of one workgroup, fixed for the whole K loop. Tile instruction
// t of wave w (of NW) copies tile rows 8 (NW t + w) .. +7; lane L fills LDS row (L / 8),
// physical chunk (L % 8), i.e. it loads the logical chunk that swz_chunk maps there (the
// map is an involution). The activation-scale instruction of wave w copies rows
// 64 (w % SA_INSTR) .. +63, the weight-scale instruction the scales of the tile's N-blocks
// (lane = N-block); waves beyond those repeat identical copies, so every wave issues the
// same INSTR_PER_WAVE vector-memory instructions per slice. Rows past M or N (and N-blocks
// past the last) lie outside their buffer resource: they read as zero and only feed outputs
// that are never stored.
// VARIANT makes the type unique to each kernel instantiation: when kernels of different
// variants shared one DmaPlan type, the host compiler emitted a launch stub for only one of them.
template <int BM, int BN, int NSTAGE, int NW, int VARIANT>
struct DmaPlan {
    using S = GemmSmem<BM, BN, NSTAGE, NW>;
    rsrc_t ra, rw, rsa, rsw;
    uint32_t a_off[S::A_INSTR], w_off[S::W_INSTR], sa_off, sw_off;

    __device__ __forceinline__ DmaPlan(int wave, int lane, const uint8_t *aq, const uint8_t *wq, const float *sa,
                                       const float *sw, int64_t m0, int64_t n0, int64_t M, int64_t N, int64_t K,
                                       int64_t nkb) {
        const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
        const int64_t rows_w = (N - n0) < BN ? (N - n0) : BN;
        ra = make_rsrc(aq + m0 * K, rows_a * K);
        rw = make_rsrc(wq + n0 * K, rows_w * K);
        rsa = make_rsrc(sa + m0 * nkb, rows_a * nkb * 4);
        const int64_t nb0 = n0 / G_SLICE, nnb = (N + G_SLICE - 1) / G_SLICE;
        rsw = make_rsrc(sw + nb0 * nkb, (nnb - nb0) * nkb * 4);
        const int sub = lane >> 3;
#pragma unroll
        for (int t = 0; t < S::A_INSTR; ++t) {
            const int row = 8 * (NW * t + wave) + sub;
            a_off[t] = (uint32_t)(row * K) + (swz_chunk(row, lane & 7) << 4);
        }
#pragma unroll
        for (int t = 0; t < S::W_INSTR; ++t) {
            const int row = 8 * (NW * t + wave) + sub;
            w_off[t] = (uint32_t)(row * K) + (swz_chunk(row, lane & 7) << 4);
        }
        sa_off = (uint32_t)((64 * (wave % S::SA_INSTR) + lane) * nkb * 4);
        sw_off = (uint32_t)(lane * nkb * 4);
    }

    // copies of slice kb into stage buffer `base`
    __device__ __forceinline__ void issue(uint8_t *base, int64_t kb, int wave) const {
        const int koff = (int)(kb * G_SLICE), soff = (int)(kb * 4);
#pragma unroll
        for (int t = 0; t < S::A_INSTR; ++t)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(base + 8 * (NW * t + wave) * G_SLICE), 16,
                                                     a_off[t], koff, 0, 0);
#pragma unroll
        for (int t = 0; t < S::W_INSTR; ++t)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(base + S::A_BYTES + 8 * (NW * t + wave) * G_SLICE),
                                                     16, w_off[t], koff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsa, (lds_void *)(base + S::A_BYTES + S::W_BYTES + (wave % S::SA_INSTR) * 256), 4, sa_off, soff, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void *)(base + S::A_BYTES + S::W_BYTES + S::SA_BYTES), 4,
                                                 sw_off, soff, 0, 0);
    }
};

template <int BM, int BN, int NW, int WAVES_M, int NSTAGE, int UNROLL, int OUT_BF16, int EXACT>
__global__ __launch_bounds__(NW * 64) void block_gemm_kernel(const uint8_t *__restrict__ aq,
                                                               const float *__restrict__ sa,
                                                               const uint8_t *__restrict__ wq,
                                                               const float *__restrict__ sw,
                                                               void *__restrict__ y, int64_t M,
                                                               int64_t N, int64_t K, int tiles_m,
                                                               int tiles_n, int group) {
    using S = GemmSmem<BM, BN, NSTAGE, NW>;
    constexpr int WAVES_N = NW / WAVES_M;
    static_assert(WAVES_M * WAVES_N == NW, "wave grid");
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;    // wave tile
    constexpr int SUB_M = WM / 16, SUB_N = WN / 16;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(S::TOTAL <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) uint8_t smem[S::TOTAL];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;

    // Tile order. Consecutive workgroups are dealt round-robin over the 8 XCDs, so
    // workgroup b (XCD b % 8, slot b / 8) is first mapped to a logical index such that each
    // XCD walks a contiguous run of logical indices: XCD x owns q + (x < rem) of them starting
    // at x*q + min(x, rem), q = tiles / 8, rem = tiles % 8 (a bijection). Logical indices
    // then run down `group` tile rows before moving one tile column right, so the tiles an
    // XCD holds at once form a compact block and share A and W panels in its L2.
    const int tiles = tiles_m * tiles_n;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int q = tiles >> 3, rem = tiles & 7;
    const int logical = xcd * q + (xcd < rem ? xcd : rem) + slot;
    const int band = logical / (group * tiles_n);                 // band of `group` tile rows
    const int in_band = logical - band * group * tiles_n;
    const int band_rows = min(group, tiles_m - band * group);
    const int tile_m = band * group + in_band % band_rows;
    const int tile_n = in_band / band_rows;
    const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;
    const int64_t nkb = K / G_SLICE;

    f32x4 acc[SUB_M][SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const DmaPlan<BM, BN, NSTAGE, NW, UNROLL * 4 + OUT_BF16 * 2 + EXACT> dma(wave, lane, aq, wq, sa, sw, m0, n0, M, N, K, nkb);
    // prologue: slices 0 .. NSTAGE-2 in flight
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
        if (st < nkb) dma.issue(smem + st * S::STAGE, st, wave);

    const int frow = lane & 15, kgroup = lane >> 4;
    // index of each n-subtile's N-block among the tile's N-blocks
    constexpr bool ONE_SW = (BN % G_SLICE == 0) && (G_SLICE % WN == 0);   // wave columns in one N-block
    int sw_idx[SUB_N];
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) sw_idx[j] = (int)(((n0 % G_SLICE) + wn * WN + 16 * j) / G_SLICE);

    // K loop; with UNROLL the stage index (and so every stage buffer offset) is a constant
    constexpr int U = UNROLL ? NSTAGE : 1;
    for (int64_t kb0 = 0; kb0 < nkb; kb0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kb = kb0 + u;
            if (kb >= nkb) break;
            const int st = UNROLL ? u : (int)(kb % NSTAGE);
            // slice kb has landed once at most (NSTAGE - 2) later slices are outstanding
            if (kb + NSTAGE - 2 < nkb) wait_vmcnt<(NSTAGE - 2) * S::INSTR_PER_WAVE>();
            else wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            // every wave has finished slice kb-1, whose buffer now receives slice kb + NSTAGE - 1
            if (kb + NSTAGE - 1 < nkb) dma.issue(smem + ((st + NSTAGE - 1) % NSTAGE) * S::STAGE, kb + NSTAGE - 1, wave);

            const uint8_t *stage = smem + st * S::STAGE;
            const uint8_t *tA = stage, *tW = stage + S::A_BYTES;
            const float *tS = reinterpret_cast<const float *>(stage + S::A_BYTES + S::W_BYTES);
            const float *tSW = reinterpret_cast<const float *>(stage + S::A_BYTES + S::W_BYTES + S::SA_BYTES);
            float swv[SUB_N];
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) swv[j] = ONE_SW ? tSW[sw_idx[0]] : tSW[sw_idx[j]];

            i32x8 wf[SUB_N];
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) wf[j] = load_frag(tW, wn * WN + 16 * j + frow, kgroup);
            Frag16 wh[EXACT ? SUB_N : 1];
            if constexpr (EXACT) {
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) wh[j] = to_f16(wf[j]);
            }
            // A fragments are read one 16-row group ahead of the MFMAs that consume them, and
            // the promotion of group i-1 is interleaved with the MFMAs of group i
            i32x8 af = load_frag(tA, wm * WM + frow, kgroup);
            float sav = tS[wm * WM + frow];
            f32x4 p_prev[SUB_N];
            float f_prev[SUB_N];
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) {
                i32x8 af_next = af;
                float sav_next = sav;
                if (i + 1 < SUB_M) {
                    af_next = load_frag(tA, wm * WM + 16 * (i + 1) + frow, kgroup);
                    sav_next = tS[wm * WM + 16 * (i + 1) + frow];
                }
                f32x4 p_cur[SUB_N];
                float f_cur[SUB_N];
                if constexpr (ONE_SW) {
                    const float f = sav * swv[0];
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) f_cur[j] = f;
                } else {
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) f_cur[j] = sav * swv[j];
                }
                if constexpr (EXACT) {
                    const Frag16 ah = to_f16(af);
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) {
                        p_cur[j] = mfma_slice_exact(wh[j], ah);
                        if (i > 0) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[i - 1][j][r] = __builtin_fmaf(p_prev[j][r], f_prev[j], acc[i - 1][j][r]);
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) {
                        p_cur[j] = mfma_slice(wf[j], af);
                        if (i > 0) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[i - 1][j][r] = __builtin_fmaf(p_prev[j][r], f_prev[j], acc[i - 1][j][r]);
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) {
                    p_prev[j] = p_cur[j];
                    f_prev[j] = f_cur[j];
                }
                af = af_next;
                sav = sav_next;
            }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[SUB_M - 1][j][r] = __builtin_fmaf(p_prev[j][r], f_prev[j], acc[SUB_M - 1][j][r]);
        }
    }

    // epilogue: lane holds Y[m][n .. n+3] for each (i, j)
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < SUB_M; ++i) {
        const int64_t m = m0 + wm * WM + 16 * i + frow;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
            const int64_t n = n0 + wn * WN + 16 * j + 4 * kgroup;
            if (n >= N) continue;
            const f32x4 v = acc[i][j];
            if constexpr (OUT_BF16) {
                uint16_t *yp = reinterpret_cast<uint16_t *>(y) + m * N + n;
                const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<u32x2 *>(yp) = u32x2{lo, hi};
                } else {
                    const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
                    for (int r = 0; r < 4 && n + r < N; ++r) yp[r] = h[r];
                }
            } else {
                float *yp = reinterpret_cast<float *>(y) + m * N + n;
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<f32x4 *>(yp) = v;
                } else {
                    for (int r = 0; r < 4 && n + r < N; ++r) yp[r] = v[r];
                }
            }
        }
    }
}

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, bool) { return 0; }

// Rows of A plus rows of W that the first concurrent tiles of one XCD touch when logical
// tiles run down `group` tile rows at a time (each XCD holds about cus_per_xcd tiles).
static int64_t xcd_panel_rows(int64_t tiles_m, int64_t tiles_n, int64_t group, int64_t bm, int64_t bn) {
    const int64_t cus_per_xcd = 32;
    const int64_t g = group < tiles_m ? group : tiles_m;
    const int64_t cols = (cus_per_xcd + g - 1) / g;
    return g * bm + (cols < tiles_n ? cols : tiles_n) * bn;
}

static int choose_group(int64_t tiles_m, int64_t tiles_n, int64_t bm, int64_t bn) {
    int best = 1;
    int64_t best_rows = xcd_panel_rows(tiles_m, tiles_n, 1, bm, bn);
    for (int g = 2; g <= 32; g *= 2) {
        const int64_t r = xcd_panel_rows(tiles_m, tiles_n, g, bm, bn);
        if (r < best_rows) {
            best_rows = r;
            best = g;
        }
    }
    return best;
}

template <int BM, int BN, int NW, int WAVES_M, int NSTAGE, int UNROLL, int EXACT>
static hipError_t launch_cfg(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, void *y,
                             bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int group = choose_group(tiles_m, tiles_n, BM, BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(NW * 64);
    if (out_bf16)
        block_gemm_kernel<BM, BN, NW, WAVES_M, NSTAGE, UNROLL, 1, EXACT><<<grid, block, 0, stream>>>(
            aq, sa, wq, sw, y, M, N, K, (int)tiles_m, (int)tiles_n, group);
    else
        block_gemm_kernel<BM, BN, NW, WAVES_M, NSTAGE, UNROLL, 0, EXACT><<<grid, block, 0, stream>>>(
            aq, sa, wq, sw, y, M, N, K, (int)tiles_m, (int)tiles_n, group);
    return hipGetLastError();
}

// Tile configurations of the FP8-matrix-unit path: (BM, BN, waves, waves along M, stages).
enum GemmTile {
    T256x128 = 0, T256x128U, T128x128, T256x128W8, T256x128W8U, T256x256W8,
    T128x192, T128x192U, T128x256W8, T128x256W8U, T_COUNT
};

static const char *const kTileNames[T_COUNT] = {"256x128",   "256x128u",  "128x128", "256x128w8",
                                                "256x128w8u", "256x256w8", "128x192", "128x192u",
                                                "128x256w8", "128x256w8u"};

// Shape -> tile. FP8Q_GEMM_TILE (one of kTileNames) overrides the choice; it exists for
// tuning and is read once.
static int choose_tile(int64_t M, int64_t N) {
    static const int forced = [] {
        const char *e = std::getenv("FP8Q_GEMM_TILE");
        if (e)
            for (int t = 0; t < T_COUNT; ++t)
                if (std::strcmp(e, kTileNames[t]) == 0) return t;
        return -1;
    }();
    if (forced >= 0) return forced;
    (void)M;
    (void)N;
    return T256x128;
}

hipError_t launch_block_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                             void *y, bool out_bf16, bool exact, int64_t M, int64_t N, int64_t K, void *, size_t,
                             hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (exact) return launch_cfg<128, 128, 4, 2, 4, 0, 1>(aq, sa, wq, sw, y, out_bf16, M, N, K, stream);
#define FP8Q_CFG(BM_, BN_, NW_, WM_, NS_, U_) \
    return launch_cfg<BM_, BN_, NW_, WM_, NS_, U_, 0>(aq, sa, wq, sw, y, out_bf16, M, N, K, stream)
    switch (choose_tile(M, N)) {
    case T256x128U: FP8Q_CFG(256, 128, 4, 2, 3, 1);
    case T128x128: FP8Q_CFG(128, 128, 4, 2, 4, 0);
    case T256x128W8: FP8Q_CFG(256, 128, 8, 4, 3, 0);
    case T256x128W8U: FP8Q_CFG(256, 128, 8, 4, 3, 1);
    case T256x256W8: FP8Q_CFG(256, 256, 8, 2, 2, 0);
    case T128x192: FP8Q_CFG(128, 192, 4, 2, 3, 0);
    case T128x192U: FP8Q_CFG(128, 192, 4, 2, 3, 1);
    case T128x256W8: FP8Q_CFG(128, 256, 8, 2, 3, 0);
    case T128x256W8U: FP8Q_CFG(128, 256, 8, 2, 3, 1);
    default: FP8Q_CFG(256, 128, 4, 2, 3, 0);
    }
#undef FP8Q_CFG
}

}  // namespace fp8q
