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
// Tiling. A workgroup of NW waves owns a BM x BN output tile (or, with split-K, one of
// `splits` contiguous K ranges of it); its waves form a WAVES_M x WAVES_N grid, each owning
// (16*SUB_M) x (16*SUB_N). Both operands are K-contiguous. Each K slice of the tile (BM + BN
// rows of 128 bytes, plus the BM activation scales and the tile's weight scales of that
// slice) is copied global -> LDS by LDS-DMA loads (buffer_load ... lds), bypassing
// registers, into one of NSTAGE stage buffers. 16-byte chunks of a row are XOR-swizzled
// (swz_chunk) so that fragment reads are free of bank conflicts. Rows past M or N lie
// outside the loads' buffer range and read as zero; they only feed outputs that are never
// stored.
//
// Schedule of one slice, per wave. The W fragments of the slice and the A fragment of the
// first 16-row group are in registers when it starts. For each row group i the A
// fragment of group i+1 is read, the SUB_N MFMAs of group i are issued, and between them
// go the promotion FMAs of the previous group (whose MFMAs have finished by then; the last
// group of a slice is promoted during the first group of the next) and a few of the copy
// instructions of slice kb + NSTAGE - 1. Scheduling barriers keep the compiler from
// regrouping these. Once per slice the wave waits for its share of the next slice's
// copies and meets the other waves at the workgroup barrier, after which the next slice is
// visible and the buffer of slice kb - 1 (now refilled during slice kb + 1) is free; then
// it reads the next slice's first fragments while MFMAs it has already issued keep the
// matrix unit busy. Tiles whose waves have registers to spare (FP8 products, 8 waves, small
// wave tiles) instead hold two slices' fragments in registers and read all of slice kb + 1
// during slice kb (the `PF` schedule in the kernel).
//
// Split-K. For shapes with too few tiles to fill the 256 CUs the K slices are divided into
// `splits` contiguous ranges. Each workgroup stores its fp32 partial tile to the caller's
// workspace and counts its arrival in the tile's arrival word; the last to arrive adds the
// partials in split order (so the result does not depend on arrival order) and writes Y.
// Arrival words carry the launch's epoch (a host counter) beside the count: a word holding
// another epoch counts as zero arrivals, so a workspace needs no clearing before its first
// use and a call that never completed leaves nothing that a later call would misread.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int G_SLICE = 128;   // K slice = promotion interval = one f8f6f4 MFMA

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ROWB: the second operand has one scale per row and slice (sw [N, K/128], the layout of
// the activation scales) instead of one per 128-row block and slice.
template <int BM, int BN, int NSTAGE, int NW, int ROWB = 0>
struct GemmSmem {
    static_assert(BM % 64 == 0 && BN % 64 == 0 && BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile shape");
    static constexpr int A_BYTES = BM * G_SLICE;
    static constexpr int W_BYTES = BN * G_SLICE;
    static constexpr int SA_BYTES = BM * 4;
    // weight scales: of 64 N-blocks from the tile's first, or (ROWB) of every tile row
    static constexpr int SW_BYTES = ROWB ? BN * 4 : 64 * 4;
    static constexpr int STAGE = A_BYTES + W_BYTES + SA_BYTES + SW_BYTES;
    static constexpr int DUMMY = STAGE * NSTAGE;   // 256-byte landing area of padding copies
    static constexpr int FLAG = DUMMY + 256;       // split-K "last to arrive" flag
    static constexpr int TOTAL = FLAG + 16;
    // LDS-DMA instructions per wave and slice: each tile instruction moves 1 KiB (8 rows of
    // 128 B), each scale instruction 256 B (64 rows of one fp32)
    static constexpr int A_INSTR = BM / (8 * NW), W_INSTR = BN / (8 * NW);
    static constexpr int SA_BLOCKS = BM / 64, SA_INSTR = (SA_BLOCKS + NW - 1) / NW;
    static constexpr int SB_BLOCKS = BN / 64, SW_INSTR = ROWB ? (SB_BLOCKS + NW - 1) / NW : 1;
    static constexpr int IPW = A_INSTR + W_INSTR + SA_INSTR + SW_INSTR;
    static_assert((NSTAGE - 1) * IPW < 64, "vmcnt range");
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

// Fragment of one 16-row group: lane l supplies row (l % 16) and, with g = l / 16, the
// 16-byte chunks g and 4 + g of the 128-byte slice (k = 16g .. 16g+15 and 64+16g .. 64+16g+15).
// Both MFMA operands use this lane -> k mapping, so matching k are paired; each 8-byte half
// of a chunk is an aligned run of 8 consecutive k. (The reads are issued in the kernel from
// per-lane offsets computed once.)

// acc += p * f per element. The empty asm consumes the result where the FMAs are written:
// without it the compiler sinks all promotions of a slice past the branches that follow
// them, keeping every slice partial live at once (and spilling).
__device__ __forceinline__ void promote(f32x4 &acc, const f32x4 &p, float f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], f, acc[r]);
    asm volatile("" : "+v"(acc));
}

// acc += p * f per element, with one factor per element (per-row scales on both operands)
__device__ __forceinline__ void promote(f32x4 &acc, const f32x4 &p, const f32x4 &f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], f[r], acc[r]);
    asm volatile("" : "+v"(acc));
}

// wait for every outstanding LDS read (lgkmcnt 0; vmcnt and expcnt left alone)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt encoding on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until the copies of a slice have landed, given that `later` slices were
// queued after it (vector-memory loads retire in issue order, IPW instructions per slice).
template <int IPW, int L>
__device__ __forceinline__ void wait_slice(int later) {
    if constexpr (L == 0) {
        wait_vmcnt<0>();
    } else {
        if (later >= L) wait_vmcnt<L * IPW>();
        else wait_slice<IPW, L - 1>(later);
    }
}

// Workgroup barrier that orders LDS traffic: the LDS-DMA copies a wave waited for (vmcnt)
// and the fragment reads it finished before the barrier, against reads and copies after.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// cache policy of buffer loads and stores: sc1 = device scope (coherent across the XCDs'
// separate L2 caches)
constexpr int kDeviceScope = 16;

// Buffer resource over `bytes` bytes at p (raw buffer, 32-bit offsets). Loads at offsets
// >= bytes return zero instead of touching memory.
__device__ __forceinline__ rsrc_t make_rsrc(const void *p, int64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}

// Per-lane LDS-DMA offsets of one workgroup, fixed for the whole K loop. Tile instruction
// t of wave w (of NW) copies tile rows 8 (NW t + w) .. +7; lane L fills LDS row (L / 8),
// physical chunk (L % 8), i.e. it loads the logical chunk that swz_chunk maps there (the
// map is an involution). Activation-scale instruction t of wave w copies rows 64 b .. +63,
// b = NW t + w; where b >= BM / 64 the instruction only pads the count (every wave issues
// the same IPW vector-memory instructions per slice) and reads one line into a dummy LDS
// area. The weight-scale instruction copies the scales of the (at most 3) N-blocks the tile
// spans, lane = N-block; the other lanes repeat lane 0's address, so they add no line
// requests. (Each scale instruction addresses one line per active distinct row, so these
// paddings would otherwise cost as many line requests as the tile rows themselves.) With
// per-row weight scales (ROWB) the weight-scale instructions copy 64 tile rows each, like
// the activation-scale instructions.
// VARIANT makes the type unique to each kernel instantiation: when kernels of different
// variants shared one DmaPlan type, the host compiler emitted a launch stub for only one of them.
template <int BM, int BN, int NSTAGE, int NW, int VARIANT, int NG, int ROWB>
struct DmaPlan {
    using S = GemmSmem<BM, BN, NSTAGE, NW, ROWB>;
    rsrc_t ra, rw, rsa, rsw;
    uint32_t off[S::IPW];
    int w;
    int sa_step;   // bytes between the activation scales of consecutive K slices
    uint8_t *dummy;

    // sa_ld: 0 for row-major activation scales [M, nkb], else the row count of K-block-major
    // scales [nkb, sa_ld] (one slice's scales of consecutive rows contiguous)
    __device__ __forceinline__ DmaPlan(int wave, int lane, const uint8_t *aq, const uint8_t *wq, const float *sa,
                                       const float *sw, int64_t m0, int64_t n0, int64_t M, int64_t N, int64_t K,
                                       int64_t nkb, int64_t sa_ld, uint8_t *smem_dummy) {
        const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
        const int64_t rows_w = (N - n0) < BN ? (N - n0) : BN;
        ra = make_rsrc(aq + m0 * K, rows_a * K);
        rw = make_rsrc(wq + n0 * K, rows_w * K);
        // K-block-major: rows past M of a tile read the next slice's first scales (or, in
        // the last slice, zero); they only feed outputs that are never stored
        if (sa_ld) {
            rsa = make_rsrc(sa + m0, (nkb * sa_ld - m0) * 4);
            sa_step = (int)(sa_ld * 4);
        } else {
            rsa = make_rsrc(sa + m0 * nkb, rows_a * nkb * 4);
            sa_step = 4;
        }
        const int sa_row = sa_ld ? 4 : (int)(nkb * 4);
        if constexpr (ROWB) {
            rsw = make_rsrc(sw + n0 * nkb, rows_w * nkb * 4);
        } else {
            const int64_t nb0 = n0 / G_SLICE, nnb = (N + G_SLICE - 1) / G_SLICE;
            rsw = make_rsrc(sw + nb0 * nkb, (nnb - nb0) * nkb * 4);
        }
        w = wave;
        dummy = smem_dummy;
        const int sub = lane >> 3;
#pragma unroll
        for (int t = 0; t < S::A_INSTR; ++t) {
            const int row = 8 * (NW * t + w) + sub;
            off[t] = (uint32_t)(row * K) + (swz_chunk(row, lane & 7) << 4);
        }
#pragma unroll
        for (int t = 0; t < S::W_INSTR; ++t) {
            const int row = 8 * (NW * t + w) + sub;
            off[S::A_INSTR + t] = (uint32_t)(row * K) + (swz_chunk(row, lane & 7) << 4);
        }
#pragma unroll
        for (int t = 0; t < S::SA_INSTR; ++t) {
            const int b = NW * t + w;
            off[S::A_INSTR + S::W_INSTR + t] = b < S::SA_BLOCKS ? (uint32_t)((64 * b + lane) * sa_row) : 0u;
        }
        if constexpr (ROWB) {
#pragma unroll
            for (int t = 0; t < S::SW_INSTR; ++t) {
                const int b = NW * t + w;
                off[S::IPW - S::SW_INSTR + t] = b < S::SB_BLOCKS ? (uint32_t)((64 * b + lane) * nkb * 4) : 0u;
            }
        } else {
            off[S::IPW - 1] = (uint32_t)((lane < 4 ? lane : 0) * nkb * 4);
        }
    }

    // instruction I (of IPW) of the copies of slice kb into stage buffer `base`; I is a
    // constant wherever this is inlined (the loops that call it are unrolled)
    __device__ __forceinline__ void issue_one(uint8_t *base, int koff, int soff, int saoff, int I) const {
        if (I < S::A_INSTR) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(base + 8 * (NW * I + w) * G_SLICE), 16, off[I],
                                                     koff, 0, 0);
        } else if (I < S::A_INSTR + S::W_INSTR) {
            const int t = I - S::A_INSTR;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(base + S::A_BYTES + 8 * (NW * t + w) * G_SLICE),
                                                     16, off[I], koff, 0, 0);
        } else if (I < S::IPW - S::SW_INSTR) {
            const int b = NW * (I - S::A_INSTR - S::W_INSTR) + w;
            uint8_t *dst = b < S::SA_BLOCKS ? base + S::A_BYTES + S::W_BYTES + b * 256 : dummy;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void *)dst, 4, off[I], saoff, 0, 0);
        } else if (ROWB) {
            const int b = NW * (I - (S::IPW - S::SW_INSTR)) + w;
            uint8_t *dst = b < S::SB_BLOCKS ? base + S::A_BYTES + S::W_BYTES + S::SA_BYTES + b * 256 : dummy;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void *)dst, 4, off[I], soff, 0, 0);
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void *)(base + S::A_BYTES + S::W_BYTES + S::SA_BYTES),
                                                     4, off[I], soff, 0, 0);
        }
    }

    // all copies of slice kb into stage buffer `base`
    __device__ __forceinline__ void issue(uint8_t *base, int64_t kb) const {
        const int koff = __builtin_amdgcn_readfirstlane((int)(kb * G_SLICE));
        const int soff = __builtin_amdgcn_readfirstlane((int)(kb * 4));
        const int saoff = __builtin_amdgcn_readfirstlane((int)kb * sa_step);
#pragma unroll
        for (int I = 0; I < S::IPW; ++I) issue_one(base, koff, soff, saoff, I);
    }

    // part g of NG (g a constant after unrolling) of the copies of slice kb: instructions
    // [g * PER, min((g + 1) * PER, IPW)), PER = ceil(IPW / NG)
    __device__ __forceinline__ void issue_part(uint8_t *base, int64_t kb, int g) const {
        constexpr int PER = (S::IPW + NG - 1) / NG;
        // kb is the same in every lane; saying so keeps the offsets in SGPRs (a VGPR soffset
        // would make the compiler wrap each copy in a per-value loop)
        const int koff = __builtin_amdgcn_readfirstlane((int)(kb * G_SLICE));
        const int soff = __builtin_amdgcn_readfirstlane((int)(kb * 4));
        const int saoff = __builtin_amdgcn_readfirstlane((int)kb * sa_step);
#pragma unroll
        for (int c = 0; c < PER; ++c)
            if (g * PER + c < S::IPW) issue_one(base, koff, soff, saoff, g * PER + c);
    }
};

// Kernel arguments (one struct so that every tile variant has the same signature).
struct GemmArgs {
    const uint8_t *aq;
    const float *sa;
    const uint8_t *wq;
    const float *sw;
    void *y;
    const float *bias;  // [N] fp32 added to every row before the output rounding, or null
    float *part;        // split-K partial tiles [splits][tiles][BM * BN], or null
    uint64_t *count;    // split-K arrival word per tile: (epoch << 32) | arrivals
    uint32_t epoch;     // this launch's epoch (non-zero)
    // grouped (per-expert) GEMM: expert e owns rows [offsets[e], offsets[e+1]) of A and Y and
    // the weight wq + e*N*K (scales sw + e*ceil(N/128)*K/128); null for a plain GEMM
    const int64_t *offsets;
    int64_t M, N, K;
    int tiles_m, tiles_n, group, splits;
    int experts;
    int sa_kmajor;      // plain GEMM: sa is K-block-major [K/128, M] (M * K/128 < 2^29)
};

constexpr int kMaxExperts = (int)kMaxGroupedExperts;

// Grouped GEMM work decode, run by the whole workgroup. Expert e has c_e = ceil(rows_e / BM)
// m-tiles; its c_e * tiles_n tiles are numbered consecutively, experts in order, and within
// an expert the m-tile varies fastest, so the tiles that read the same weight panel are
// adjacent. The numbers are dealt to the XCDs in contiguous runs (as in the plain GEMM) over
// the real tile count, so surplus workgroups of the upper-bound grid are spread evenly and
// the XCDs get equal shares. Returns false for a workgroup with no tile. Uses `scratch`
// (LDS, at least 4 * (kMaxExperts + 1) + 16 bytes) and synchronises the workgroup. Only the
// grouped kernel instantiations contain it, so it does not weigh on the plain GEMM's
// registers.
template <int BM, int NT>
__device__ __forceinline__ bool grouped_tile(const GemmArgs &g, uint8_t *scratch, int &expert, int64_t &row0,
                                             int64_t &row1, int &tile_n) {
    int *prefix = reinterpret_cast<int *>(scratch);            // m-tiles before expert e
    int *found = prefix + kMaxExperts + 1;
    const int E = g.experts;
    // per-expert m-tile counts; rows are clamped to [0, M] so that any offsets stay in bounds
    constexpr int PER = (kMaxExperts + NT - 1) / NT;
    const int e0 = threadIdx.x * PER;
    int local[PER], sum = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = e0 + u;
        int c = 0;
        if (e < E) {
            int64_t r0 = g.offsets[e], r1 = g.offsets[e + 1];
            r0 = r0 < 0 ? 0 : (r0 > g.M ? g.M : r0);
            r1 = r1 < r0 ? r0 : (r1 > g.M ? g.M : r1);
            c = (int)((r1 - r0 + BM - 1) / BM);
        }
        local[u] = sum;
        sum += c;
    }
    // exclusive scan of the per-thread sums (Hillis-Steele in LDS)
    prefix[threadIdx.x] = sum;
    __syncthreads();
    for (int d = 1; d < NT; d <<= 1) {
        const int v = threadIdx.x >= d ? prefix[threadIdx.x - d] : 0;
        __syncthreads();
        prefix[threadIdx.x] += v;
        __syncthreads();
    }
    const int before = threadIdx.x > 0 ? prefix[threadIdx.x - 1] : 0;
    const int total = prefix[NT - 1];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u)
        if (e0 + u <= E) prefix[e0 + u] = before + local[u];
    if (threadIdx.x == 0) prefix[E] = total;
    __syncthreads();
    // XCD x (workgroups b with b % 8 == x) takes logical tiles [x*q + min(x, rem), +q + (x < rem))
    const int units = total * g.tiles_n;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int q = units >> 3, rem = units & 7;
    if (slot >= q + (xcd < rem ? 1 : 0)) return false;
    const int logical = xcd * q + (xcd < rem ? xcd : rem) + slot;
    // the expert whose tile numbers [prefix[e] * tiles_n, prefix[e+1] * tiles_n) hold
    // `logical` (several threads search disjoint parts; exactly one match)
    for (int e = threadIdx.x; e < E; e += NT)
        if (prefix[e] * g.tiles_n <= logical && logical < prefix[e + 1] * g.tiles_n) *found = e;
    __syncthreads();
    expert = *found;
    const int first = prefix[expert], cnt = prefix[expert + 1] - first;
    const int in_expert = logical - first * g.tiles_n;
    tile_n = in_expert / cnt;
    int64_t r0 = g.offsets[expert], r1 = g.offsets[expert + 1];
    r0 = r0 < 0 ? 0 : (r0 > g.M ? g.M : r0);
    r1 = r1 < r0 ? r0 : (r1 > g.M ? g.M : r1);
    row0 = r0 + (int64_t)(in_expert - tile_n * cnt) * BM;
    row1 = r1;
    __syncthreads();   // the scratch is reused by the caller
    return true;
}

template <int BM, int BN, int NW, int WAVES_M, int NSTAGE, int OUT_BF16, int EXACT, int GROUPED, int ROWB>
__global__ __launch_bounds__(NW * 64) void block_gemm_kernel(GemmArgs g) {
    static_assert(!(GROUPED && ROWB), "per-row weight scales are not grouped");
    using S = GemmSmem<BM, BN, NSTAGE, NW, ROWB>;
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

    // Work order. Consecutive workgroups are dealt round-robin over the 8 XCDs, so
    // workgroup b (XCD b % 8, slot b / 8) is first mapped to a logical index such that each
    // XCD walks a contiguous run of logical indices: XCD x owns q + (x < rem) of them starting
    // at x*q + min(x, rem), q = units / 8, rem = units % 8 (a bijection). The split index is
    // the slowest-varying part of the logical index; within one split, logical tiles run down
    // `group` tile rows before moving one tile column right, so the tiles an XCD holds at
    // once form a compact block and share A and W panels in its L2.
    const int64_t N = g.N, K = g.K;
    const int64_t nkb = K / G_SLICE;
    const uint8_t *wq = g.wq;
    const float *sw = g.sw;
    int split = 0, tl = 0;
    int64_t m0, n0, M;   // first row and column of the tile; M: end of its row range
    if constexpr (!GROUPED) {
        const int tiles = g.tiles_m * g.tiles_n;
        const int units = tiles * g.splits;
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int q = units >> 3, rem = units & 7;
        const int logical = xcd * q + (xcd < rem ? xcd : rem) + slot;
        split = logical / tiles;
        tl = logical - split * tiles;
        const int band = tl / (g.group * g.tiles_n);             // band of `group` tile rows
        const int in_band = tl - band * g.group * g.tiles_n;
        const int band_rows = min(g.group, g.tiles_m - band * g.group);
        const int tile_m = band * g.group + in_band % band_rows;
        const int tile_n = in_band / band_rows;
        m0 = (int64_t)tile_m * BM;
        n0 = (int64_t)tile_n * BN;
        M = g.M;
    } else {
        // grouped: the grid is an upper bound on the tiles of all experts; surplus
        // workgroups exit
        int expert, tile_n;
        int64_t r0, r1;
        if (!grouped_tile<BM, NW * 64>(g, smem, expert, r0, r1, tile_n)) return;
        m0 = r0;
        M = r1;
        n0 = (int64_t)tile_n * BN;
        wq += (int64_t)expert * N * K;
        sw += (int64_t)expert * ((N + G_SLICE - 1) / G_SLICE) * nkb;
    }
    const int64_t kb0 = split * nkb / g.splits, kb1 = (split + 1) * nkb / g.splits;

    f32x4 acc[SUB_M][SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15, kgroup = lane >> 4;
    // index of each n-subtile's N-block among the tile's N-blocks
    constexpr bool ONE_SW = (BN % G_SLICE == 0) && (G_SLICE % WN == 0);   // wave columns in one N-block
    int sw_idx[SUB_N];
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) sw_idx[j] = (int)(((n0 % G_SLICE) + wn * WN + 16 * j) / G_SLICE);

    if (kb0 < kb1) {
        // Where the slice barrier sits. With three or more stages the copies have slack, and
        // the barrier goes before the last row group: that group's MFMAs (operands already in
        // registers) then run while the next slice's first fragments are read. With two
        // stages the next slice's copies have only one slice of lead, and the barrier goes
        // after the last group's MFMAs, as late as possible (measured: 4% faster there).
        constexpr bool EARLY_BARRIER = NSTAGE >= 3;
        // Whole-slice register prefetch (see below): FP8 products, 8 waves, and only where two
        // register sets of a slice's fragments fit beside the accumulators.
        constexpr bool PF = NW == 8 && !EXACT && !ROWB && SUB_M >= 2 && NSTAGE >= 3 &&
                            (SUB_M + SUB_N) * 16 + SUB_M * SUB_N * 4 <= 192;
        // The copies queued during a slice are spread over the row groups that run before its
        // barrier (all of them with the late barrier), so that at the barrier every slice
        // queued after the next one is complete in the vector-memory count and the count
        // wait of wait_slice covers exactly the next slice.
        // Each MFMA slot of those row groups issues at most one copy instruction: a wave whose
        // copy waits for the address unit stalls its in-order issue, MFMAs included.
        constexpr int COPY_GROUPS = EARLY_BARRIER || PF ? SUB_M - 1 : SUB_M;
        static_assert(COPY_GROUPS >= 1, "row groups per wave");
        constexpr int COPY_PARTS = COPY_GROUPS * SUB_N;
        const DmaPlan<BM, BN, NSTAGE, NW, ROWB * 8 + GROUPED * 4 + OUT_BF16 * 2 + EXACT, COPY_PARTS, ROWB> dma(wave, lane, g.aq, wq, g.sa, sw, m0, n0, M, N,
                                                                   K, nkb, GROUPED || !g.sa_kmajor ? 0 : M, smem + S::DUMMY);
        // prologue: the first NSTAGE slices in flight
#pragma unroll
        for (int st = 0; st < NSTAGE; ++st)
            if (kb0 + st < kb1) dma.issue(smem + st * S::STAGE, kb0 + st);
        wait_slice<S::IPW, NSTAGE - 1>((int)min64(NSTAGE, kb1 - kb0) - 1);
        lds_barrier();

        // LDS byte offsets, within a stage buffer, of this lane's fragment reads and scales.
        // The rows a wave reads are (wave base) + 16 x (group) + frow with both bases multiples
        // of 16, so every fragment row has the swizzle of frow and its two chunk addresses are
        // a per-lane offset plus a constant. The empty asm pins each offset in a VGPR computed
        // once: every read is then (VGPR offset) + (compile-time stage and group offset).
        const int frag_lo = frow * G_SLICE + (swz_chunk(frow, kgroup) << 4);
        const int frag_hi = frow * G_SLICE + (swz_chunk(frow, 4 + kgroup) << 4);
        int a_lo = wm * WM * G_SLICE + frag_lo, a_hi = wm * WM * G_SLICE + frag_hi;
        int w_lo = S::A_BYTES + wn * WN * G_SLICE + frag_lo, w_hi = S::A_BYTES + wn * WN * G_SLICE + frag_hi;
        int sa_at = S::A_BYTES + S::W_BYTES + (wm * WM + frow) * 4;
        // weight scale of each n-subtile: of its N-block, or (ROWB) of this lane's four columns
        int sw_at[SUB_N];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j)
            sw_at[j] = S::A_BYTES + S::W_BYTES + S::SA_BYTES +
                       (ROWB ? (wn * WN + 16 * j + 4 * kgroup) * 4 : sw_idx[ONE_SW ? 0 : j] * 4);
        if constexpr (NW == 8) {   // (the 4-wave tiles are short of registers: offsets recomputed there)
            asm volatile("" : "+v"(a_lo), "+v"(a_hi), "+v"(w_lo), "+v"(w_hi), "+v"(sa_at));
#pragma unroll
            for (int j = 0; j < (ONE_SW && !ROWB ? 1 : SUB_N); ++j) asm volatile("" : "+v"(sw_at[j]));
        }
        auto frag_at = [&](const uint8_t *base, int lo, int hi) __device__ __attribute__((always_inline)) {
            const u32x4 l = *reinterpret_cast<const u32x4 *>(base + lo);
            const u32x4 h = *reinterpret_cast<const u32x4 *>(base + hi);
            return i32x8{(int)l.x, (int)l.y, (int)l.z, (int)l.w, (int)h.x, (int)h.y, (int)h.z, (int)h.w};
        };
        auto f32_at = [&](const uint8_t *base, int off) __device__ __attribute__((always_inline)) {
            return *reinterpret_cast<const float *>(base + off);
        };
        // weight scale(s) of n-subtile j: one float, or (ROWB) the four of this lane's columns
        using WScale = std::conditional_t<ROWB != 0, f32x4, float>;
        constexpr bool ONE_WS = ONE_SW && !ROWB;
        auto ws_at = [&](const uint8_t *base, int j) __device__ __attribute__((always_inline)) {
            if constexpr (ROWB != 0)
                return *reinterpret_cast<const f32x4 *>(base + sw_at[j]);
            else
                return *reinterpret_cast<const float *>(base + sw_at[ONE_WS ? 0 : j]);
        };

        if constexpr (PF) {
            // Whole-slice register prefetch. Two register sets hold the fragments and scales of
            // two slices: the MFMAs of slice kb take their operands from one set while the other
            // is filled from LDS with slice kb + 1, so every LDS read has most of a slice of MFMA
            // work to land behind. A stage buffer is free as soon as its slice has been read into
            // registers, which is one slice earlier than when fragments are read as they are
            // used, and the copies of slice kb + NSTAGE go into the buffer of slice kb.
            // Per slice and wave: row group 0's MFMAs; the count waits for the rest of slice kb's
            // reads and for slice kb + 1's copies, and the workgroup barrier (after which slice
            // kb + 1 is visible and every wave has finished reading slice kb); then row groups
            // 1 .. SUB_M - 1, whose MFMA slots also issue the reads of slice kb + 1 and the
            // copies of slice kb + NSTAGE. Promotion runs one row group behind its MFMAs (the last
            // group of a slice is promoted during the first group of the next).
            static_assert(SUB_M >= 2, "register prefetch needs two row groups");
            i32x8 fa[2][SUB_M], fw[2][SUB_N];
            float sa_r[2][SUB_M];
            WScale sw_r[2][SUB_N];
            constexpr int NSW = ONE_WS ? 1 : SUB_N;
            // read item `it` of a slice into register set rs: the SUB_N W fragments, then the
            // scales, then the SUB_M A fragments (the order the slice's first row group uses them)
            constexpr int ITEMS = SUB_N + 1 + SUB_M;
            constexpr int SLOTS = (SUB_M - 1) * SUB_N;
            constexpr int IPS = (ITEMS + SLOTS - 1) / SLOTS;   // read items per MFMA slot
            auto read_item = [&](const uint8_t *stage, auto rs_c, auto it_c) __device__ __attribute__((always_inline)) {
                constexpr int RS = decltype(rs_c)::value, IT = decltype(it_c)::value;
                if constexpr (IT < SUB_N) {
                    fw[RS][IT] = frag_at(stage + 16 * IT * G_SLICE, w_lo, w_hi);
                } else if constexpr (IT == SUB_N) {
#pragma unroll
                    for (int i = 0; i < SUB_M; ++i) sa_r[RS][i] = f32_at(stage + 16 * i * 4, sa_at);
#pragma unroll
                    for (int j = 0; j < NSW; ++j) sw_r[RS][j] = ws_at(stage, j);
                } else if constexpr (IT < ITEMS) {
                    fa[RS][IT - SUB_N - 1] = frag_at(stage + 16 * (IT - SUB_N - 1) * G_SLICE, a_lo, a_hi);
                }
            };
            f32x4 p_prev[SUB_N];
            WScale f_prev[SUB_N];
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
                p_prev[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                f_prev[j] = WScale{};
            }
            const int kbs = __builtin_amdgcn_readfirstlane((int)kb0);
            const int kbe = __builtin_amdgcn_readfirstlane((int)kb1);
            // slice kb uses stage (kb - kbs) % NSTAGE and register set (kb - kbs) % 2; the loop
            // is unrolled by a multiple of both, so each is a constant in each unrolled copy
            auto at = [&](int st) __device__ __attribute__((always_inline)) { return smem + (st % NSTAGE) * S::STAGE; };
            const std::integral_constant<int, 0> set0;
            static_for<ITEMS>([&](auto it) __device__ __attribute__((always_inline)) { read_item(at(0), set0, it); });
            auto step = [&](auto t_c, const int kb, auto steady_c) __device__ __attribute__((always_inline)) {
                constexpr int T = decltype(t_c)::value;
                constexpr bool STEADY = decltype(steady_c)::value;
                constexpr int R = T & 1;
                const std::integral_constant<int, R ^ 1> set_next;
                const bool more = STEADY || kb + 1 < kbe;
                const bool copy_now = STEADY || kb + NSTAGE < kbe;
                const int later = STEADY ? NSTAGE - 2 : min(NSTAGE - 2, kbe - 2 - kb);
                const uint8_t *next = at(T + 1);
                uint8_t *copy_dst = at(T);
                // (the compiler waits for each register of set R as its first MFMA needs it)
                static_for<SUB_M>([&](auto i_c) __device__ __attribute__((always_inline)) {
                    constexpr int I = decltype(i_c)::value;
                    constexpr int IP = I == 0 ? SUB_M - 1 : I - 1;   // row group being promoted
                    WScale f_cur[SUB_N];
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) f_cur[j] = sa_r[R][I] * sw_r[R][ONE_WS ? 0 : j];
                    f32x4 p_cur[SUB_N];
                    static_for<SUB_N>([&](auto j_c) __device__ __attribute__((always_inline)) {
                        constexpr int J = decltype(j_c)::value;
                        p_cur[J] = mfma_slice(fw[R][J], fa[R][I]);
                        if constexpr (I >= 1) {
                            if (copy_now) dma.issue_part(copy_dst, kb + NSTAGE, (I - 1) * SUB_N + J);
                            if (more)
                                static_for<IPS>([&](auto u_c) __device__ __attribute__((always_inline)) {
                                    read_item(next, set_next,
                                              std::integral_constant<int, ((I - 1) * SUB_N + J) * IPS + decltype(u_c)::value>{});
                                });
                        }
                        promote(acc[IP][J], p_prev[J], f_prev[J]);
                        __builtin_amdgcn_sched_barrier(0);
                    });
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) {
                        p_prev[j] = p_cur[j];
                        f_prev[j] = f_cur[j];
                    }
                    if constexpr (I == 0) {
                        if (more) {
                            // every read of slice kb has landed before the barrier that frees its buffer
                            wait_lgkm0();
                            wait_slice<S::IPW, NSTAGE - 2>(later);
                            lds_barrier();
                        }
                    }
                });
            };
            const std::false_type general;
            const std::true_type steady;
            constexpr int U = NSTAGE % 2 == 0 ? NSTAGE : 2 * NSTAGE;
            int kb = kbs;
            for (; kb + U - 1 + NSTAGE < kbe; kb += U)
                static_for<U>([&](auto t) __device__ __attribute__((always_inline)) { step(t, kb + decltype(t)::value, steady); });
            // the last (at most U - 1 + NSTAGE) slices
            static_for<U - 1 + NSTAGE>([&](auto t) __device__ __attribute__((always_inline)) {
                if (kb + decltype(t)::value < kbe) step(t, kb + decltype(t)::value, general);
            });
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) promote(acc[SUB_M - 1][j], p_prev[j], f_prev[j]);
        } else {
            // Promotion lag. A row group's SUB_N slice partials are normally promoted during the
            // next row group's MFMAs. A wave tile of 32 or more blocks (the exact-slice 256x256
            // tile, 128x64 per wave) has no registers for them beside its accumulators, so there
            // each block's partial is promoted during the next block's MFMAs, and a row group's
            // last one during the next row group's first block: one partial is carried instead
            // of SUB_N. Each output's promotions keep their slice order either way, so the
            // result is the same bit for bit.
            constexpr bool CARRY_ONE = EXACT && SUB_M * SUB_N >= 32;
            // fragments of the slice being contracted
            i32x8 wf[SUB_N];
            Frag16 wh[EXACT ? SUB_N : 1];
            WScale swv[SUB_N];
            i32x8 af;
            float sav;
            auto load_slice_head = [&](const uint8_t *stage) __device__ __attribute__((always_inline)) {
    #pragma unroll
                for (int j = 0; j < SUB_N; ++j) wf[j] = frag_at(stage + 16 * j * G_SLICE, w_lo, w_hi);
                af = frag_at(stage, a_lo, a_hi);
                sav = f32_at(stage, sa_at);
    #pragma unroll
                for (int j = 0; j < SUB_N; ++j) swv[j] = ws_at(stage, j);
                if constexpr (EXACT) {
    #pragma unroll
                    for (int j = 0; j < SUB_N; ++j) wh[j] = to_f16(wf[j]);
                }
            };
            load_slice_head(smem);

            // promotion of each row group runs one group behind its MFMAs (the last group of a
            // slice is promoted during the first group of the next); it starts from a zero partial
            f32x4 p_prev[SUB_N];
            WScale f_prev[SUB_N];
    #pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
                p_prev[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                f_prev[j] = WScale{};
            }
            // With 8 waves the K loop is unrolled by NSTAGE: each slice's stage buffer, the buffer
            // its copies go to and the next slice's buffer are then compile-time offsets, so
            // fragment reads use fixed addresses and the loop carries no stage index. (The 4-wave
            // tiles hold twice the accumulators per wave; unrolled, they run out of registers, so
            // they keep a rolled loop with a stage index.) The slice indices are wave-uniform
            // 32-bit values, which keeps the copy and barrier conditions scalar.
            const int kbs = __builtin_amdgcn_readfirstlane((int)kb0);
            const int kbe = __builtin_amdgcn_readfirstlane((int)kb1);
            // slice kb in `stage`, whose copies (slice kb + NSTAGE - 1) go to `copy_dst`, followed
            // by the slice in `next`. A steady slice (not the first, and at least NSTAGE - 1 slices
            // before the end) always queues copies and always has a successor: its body has no
            // branches.
            auto slice = [&](const uint8_t *stage, uint8_t *copy_dst, const uint8_t *next, const int kb, auto steady_c)
                             __device__ __attribute__((always_inline)) {
                constexpr bool STEADY = decltype(steady_c)::value;
                const bool more = STEADY || kb + 1 < kbe;
                const int later = STEADY ? NSTAGE - 2 : min(NSTAGE - 2, kbe - 2 - kb);
                // the copies of slice kb + NSTAGE - 1 go into the buffer of slice kb - 1, free since
                // the barrier that ended slice kb - 1; they are spread over this slice's row groups
                // so that the matrix unit is never left waiting behind a burst of copy issues
                const bool copy_now = STEADY || (kb > kbs && kb + NSTAGE - 1 < kbe);
    #pragma unroll
                for (int i = 0; i < SUB_M; ++i) {
                    // With the early barrier, the next slice's first fragments and scales are read
                    // right after it, while this slice's last row group runs on the matrix unit:
                    // each W fragment register is refilled as soon as its last MFMA has taken it.
                    const bool head_now = EARLY_BARRIER && i == SUB_M - 1 && more;
                    i32x8 af_n = af;
                    float sav_n = sav;
                    if (head_now) {
                        // every LDS read of slice kb is done (the last group's operands are in
                        // registers); once all waves are past the barrier the next slice has landed
                        wait_lgkm0();
                        wait_slice<S::IPW, NSTAGE - 2>(later);
                        lds_barrier();
                        af_n = frag_at(next, a_lo, a_hi);
                        sav_n = f32_at(next, sa_at);
                    } else if (i + 1 < SUB_M) {
                        af_n = frag_at(stage + 16 * (i + 1) * G_SLICE, a_lo, a_hi);
                        sav_n = f32_at(stage + 16 * (i + 1) * 4, sa_at);
                    }
                    WScale f_cur[SUB_N];
    #pragma unroll
                    for (int j = 0; j < SUB_N; ++j) f_cur[j] = sav * swv[ONE_WS ? 0 : j];
                    if (head_now) {
    #pragma unroll
                        for (int j = 0; j < SUB_N; ++j) swv[j] = ws_at(next, j);
                    }
                    f32x4 p_cur[SUB_N];
                    const int ip = i == 0 ? SUB_M - 1 : i - 1;   // row group being promoted (a constant once unrolled)
                    if constexpr (EXACT) {
                        const Frag16 ah = to_f16(af);
    #pragma unroll
                        for (int j = 0; j < SUB_N; ++j) {
                            p_cur[j] = mfma_slice_exact(wh[j], ah);
                            if (copy_now && i < COPY_GROUPS) dma.issue_part(copy_dst, kb + NSTAGE - 1, i * SUB_N + j);
                            if (head_now) wf[j] = frag_at(next + 16 * j * G_SLICE, w_lo, w_hi);
                            if constexpr (CARRY_ONE) {
                                if (j > 0) promote(acc[i][j - 1], p_cur[j - 1], f_cur[j - 1]);
                                else promote(acc[ip][SUB_N - 1], p_prev[0], f_prev[0]);
                            } else {
                                promote(acc[ip][j], p_prev[j], f_prev[j]);
                            }
                            // the four f16 MFMAs interleaved with the promotion FMAs (and, in the
                            // first block, the tail of the A conversion), two VALU instructions
                            // after each MFMA (measured: 2% faster than the compiler's own order
                            // on the outlier shape; 1:1, 1:3 and one pattern per row group were
                            // not faster)
                            static_for<4>([&](auto) __device__ __attribute__((always_inline)) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // two VALU
                            });
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        if constexpr (CARRY_ONE) {   // the row group's last partial
                            p_prev[0] = p_cur[SUB_N - 1];
                            f_prev[0] = f_cur[SUB_N - 1];
                        }
                        if (head_now) {
    #pragma unroll
                            for (int j = 0; j < SUB_N; ++j) wh[j] = to_f16(wf[j]);
                        }
                    } else {
    #pragma unroll
                        for (int j = 0; j < SUB_N; ++j) {
                            p_cur[j] = mfma_slice(wf[j], af);
                            if (copy_now && i < COPY_GROUPS) dma.issue_part(copy_dst, kb + NSTAGE - 1, i * SUB_N + j);
                            if (head_now) wf[j] = frag_at(next + 16 * j * G_SLICE, w_lo, w_hi);
                            promote(acc[ip][j], p_prev[j], f_prev[j]);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                    // with the late barrier (two stages) the next slice's first fragments load after
                    // the last group's MFMAs have taken their operands, while they run
                    if (!EARLY_BARRIER && i == SUB_M - 1 && more) {
                        wait_slice<S::IPW, NSTAGE - 2>(later);
                        lds_barrier();
                        load_slice_head(next);
                    }
                    if constexpr (!CARRY_ONE) {
    #pragma unroll
                        for (int j = 0; j < SUB_N; ++j) {
                            p_prev[j] = p_cur[j];
                            f_prev[j] = f_cur[j];
                        }
                    }
                    if (i + 1 < SUB_M || head_now) {
                        af = af_n;
                        sav = sav_n;
                    }
                }
            };
            const std::false_type general;
            const std::true_type steady;
            if constexpr (NW == 8) {
                // slice kb uses stage (kb - kbs) % NSTAGE, a constant in each unrolled copy
                auto at = [&](int st) __device__ __attribute__((always_inline)) { return smem + (st % NSTAGE) * S::STAGE; };
                slice(at(0), at(NSTAGE - 1), at(1), kbs, general);
                int kb = kbs + 1;
                // whole rounds of steady slices (stages 1, 2, ..., 0)
                for (; kb + 2 * NSTAGE - 2 < kbe; kb += NSTAGE)
                    static_for<NSTAGE>([&](auto t) __device__ __attribute__((always_inline)) {
                        constexpr int st = 1 + decltype(t)::value;
                        slice(at(st), at(st + NSTAGE - 1), at(st + 1), kb + decltype(t)::value, steady);
                    });
                // the last (at most 2 NSTAGE - 2) slices
                static_for<2 * NSTAGE - 2>([&](auto t) __device__ __attribute__((always_inline)) {
                    constexpr int st = 1 + decltype(t)::value;
                    if (kb + decltype(t)::value < kbe)
                        slice(at(st), at(st + NSTAGE - 1), at(st + 1), kb + decltype(t)::value, general);
                });
            } else {
                int st = 0;
                for (int kb = kbs; kb < kbe; ++kb) {
                    const int st_next = st + 1 == NSTAGE ? 0 : st + 1;
                    const int st_copy = st == 0 ? NSTAGE - 1 : st - 1;
                    slice(smem + st * S::STAGE, smem + st_copy * S::STAGE, smem + st_next * S::STAGE, kb, general);
                    st = st_next;
                }
            }
            if constexpr (CARRY_ONE) {
                promote(acc[SUB_M - 1][SUB_N - 1], p_prev[0], f_prev[0]);
            } else {
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) promote(acc[SUB_M - 1][j], p_prev[j], f_prev[j]);
            }
        }
    }

    if (g.splits > 1) {
        // split-K: publish this split's partial tile (fragment order: one 1 KiB line per
        // (wave, i, j), lane-contiguous), then count the arrival. Ordering argument, after
        // the LLVM AMDGPU backend user guide's memory model for gfx942 (whose code sequences
        // gfx950 shares): a relaxed agent-scope atomic load, store or read-modify-write is
        // the plain instruction with the sc1 (agent scope) bit; release and acquire at agent
        // scope add only an L2 write-back before (buffer_wbl2 sc1) and an invalidate after
        // (buffer_inv sc1), which serve other, non-atomic data. Here every access to the
        // exchanged data is such an agent-scope access: the partials are stored and reloaded
        // with sc1 buffer instructions, the arrival word is an agent-scope atomic. The stores
        // have completed (vmcnt 0) before the arrival is counted, and the last workgroup
        // issues its loads only after its atomic has returned and its workgroup barrier, so
        // it reads every partial. The cache maintenance is left out on purpose: at agent
        // scope it writes back or invalidates the whole L2, which costs more than the
        // partials themselves.
        const rsrc_t rp = make_rsrc(g.part + (int64_t)tl * g.splits * (BM * BN), (int64_t)g.splits * BM * BN * 4);
        const uint32_t lane_off = (uint32_t)((wave * (SUB_M * SUB_N * 64) + lane) * 16);
        const int split_off = split * (BM * BN * 4);
#pragma unroll
        for (int i = 0; i < SUB_M; ++i)
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc[i][j]), rp,
                                                       lane_off + (i * SUB_N + j) * 1024, split_off, kDeviceScope);
        wait_vmcnt<0>();
        __syncthreads();
        int *flag = reinterpret_cast<int *>(smem + S::FLAG);
        if (threadIdx.x == 0) {
            // count this arrival: a word of another epoch (stale, or never written) is zero
            // arrivals of this one. The last arrival sets the count back to zero, so a launch
            // replayed with the same epoch (a captured graph) starts from zero as well.
            uint64_t *word = &g.count[tl];
            uint64_t cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t arrived;
            for (;;) {
                const uint32_t c = (uint32_t)(cur >> 32) == g.epoch ? (uint32_t)cur : 0u;
                const uint64_t next = ((uint64_t)g.epoch << 32) | (uint64_t)(c + 1);
                if (__hip_atomic_compare_exchange_strong(word, &cur, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)) {
                    arrived = c + 1;
                    break;
                }
            }
            const int last = arrived == (uint32_t)g.splits;
            if (last) __hip_atomic_store(word, (uint64_t)g.epoch << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *flag = last;
        }
        __syncthreads();
        if (!*flag) return;
        // the last to arrive sums the partials in split order (independent of which split
        // arrived last), one row group at a time; its own partial is taken from its registers
        // (the values it stored), the others' are loaded (the loads of a row group are all
        // issued before the first is needed)
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) {
            f32x4 t[SUB_N];
            for (int sp = 0; sp < g.splits; ++sp) {
                f32x4 v[SUB_N];
                if (sp == split) {
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) v[j] = acc[i][j];
                } else {
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j)
                        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                             rp, lane_off + (i * SUB_N + j) * 1024,
                                                             sp * (BM * BN * 4), kDeviceScope));
                }
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) t[j] = sp == 0 ? v[j] : t[j] + v[j];
            }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) acc[i][j] = t[j];
        }
    }

    // Epilogue, staged through LDS (the stage buffers are free once every wave is past the
    // K loop): the fragments of IPR row groups are written to LDS as output rows, then the
    // workgroup stores them with 16 bytes per lane, so that every store instruction writes
    // whole 128-byte pieces of output rows. The LDS row stride is padded so that both the
    // fragment writes (16 rows x 4 column groups per instruction) and the row reads are
    // free of bank conflicts.
    {
        constexpr int OB = OUT_BF16 ? 2 : 4;                 // bytes per output element
        constexpr int EPC = 16 / OB;                         // elements per 16-byte chunk
        constexpr int ROW_WORDS = BN * OB / 4;
        constexpr int TARGET = OUT_BF16 ? 8 : 16;            // row stride, in banks, mod 64
        constexpr int LDS_ROW = 4 * (ROW_WORDS + ((TARGET - ROW_WORDS) % 64 + 64) % 64);
        constexpr int RG = WAVES_M * 16;                     // tile rows of one row-group index
        constexpr int IPR0 = (S::STAGE * NSTAGE) / (RG * LDS_ROW);
        constexpr int IPR = IPR0 < SUB_M ? IPR0 : SUB_M;     // row groups per round
        static_assert(IPR >= 1, "epilogue staging does not fit");
        constexpr int CPR = BN * OB / 16;                    // 16-byte chunks per output row
        const bool vec_ok = ((N * OB) & 15) == 0;            // every output row 16-byte aligned
        // bias of this lane's four output columns of each n-subtile (zero past N)
        f32x4 bvec[SUB_N];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
            bvec[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (g.bias) {
                const int64_t n = n0 + wn * WN + 16 * j + 4 * kgroup;
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
                const int i = i0 + ii;
                if (i < SUB_M) {
                    uint8_t *rowp = smem + (ii * RG + wm * 16 + frow) * LDS_ROW;
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) {
                        const int col = wn * WN + 16 * j + 4 * kgroup;
                        const f32x4 v = acc[i][j] + bvec[j];
                        if constexpr (OUT_BF16)
                            *reinterpret_cast<u32x2 *>(rowp + col * 2) =
                                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        else
                            *reinterpret_cast<f32x4 *>(rowp + col * 4) = v;
                    }
                }
            }
            __syncthreads();
            const int groups = (SUB_M - i0) < IPR ? (SUB_M - i0) : IPR;
            const int chunks = groups * RG * CPR;
            for (int c = threadIdx.x; c < chunks; c += NW * 64) {
                const int r = c / CPR, cb = c - r * CPR;
                const int ii = r / RG, within = r - ii * RG;
                const int64_t m = m0 + (within >> 4) * WM + 16 * (i0 + ii) + (within & 15);
                const int64_t n = n0 + cb * EPC;
                if (m >= M || n >= N) continue;
                const uint8_t *src = smem + r * LDS_ROW + cb * 16;
                uint8_t *yp = reinterpret_cast<uint8_t *>(g.y) + (m * N + n) * OB;
                if (vec_ok && n + EPC <= N) {
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(src), reinterpret_cast<u32x4 *>(yp));
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

// ---------------------------------------------------------------------------------------
// host side: tile and split choice, workspace, launch

// Tile configurations: (BM, BN, waves, waves along M, stages). The timing columns are
// measured on MI355X (bf16 output, 512 tiles on 256 CUs, K = 1024 and 4096), per
// contraction mode: the duration of one K slice of one tile, and the fixed cost of a tile
// (first copies in flight, output stores). The exact-slice columns of 256x256w8 were measured
// later on one box beside 256x128w8, 128x256w8 and 128x192w8 (fp32 output, same shapes) and
// scaled by the ratio of those three tiles' slice times to their columns here.
enum GemmTile {
    T256x256W8 = 0, T256x192W8, T256x128W8, T128x256W8, T128x192W8, T256x128, T128x128, T128x128S2,
    T_COUNT
};

struct TileInfo {
    const char *name;
    int bm, bn;
    bool fp8_ok, exact_ok;
    double us_slice, us_fixed;       // FP8-product mode
    double us_slice_x, us_fixed_x;   // exact-slice mode (0: not implemented)
    int rowb_ok;                     // instantiated with per-row weight scales: 1 FP8 mode, 2 exact mode
};

static const TileInfo kTiles[T_COUNT] = {
    {"256x256w8", 256, 256, true, true, 1.74, 11.1, 3.73, 13.4, 0},
    {"256x192w8", 256, 192, true, false, 1.51, 7.1, 0, 0, 0},
    {"256x128w8", 256, 128, true, true, 1.00, 7.8, 2.04, 5.9, 1},
    {"128x256w8", 128, 256, true, true, 0.91, 7.9, 2.10, 4.7, 1},
    {"128x192w8", 128, 192, true, true, 0.72, 6.2, 1.61, 4.7, 3},
    {"256x128", 256, 128, true, false, 1.24, 7.5, 0, 0, 0},
    {"128x128", 128, 128, true, true, 0.80, 5.0, 1.36, 4.6, 3},
    {"128x128s2", 128, 128, false, false, 0.95, 2.8, 0, 0, 0},
};

constexpr int kNumCUs = 256;
constexpr int kMaxSplits = 8;

// Rows of A plus rows of W that the first concurrent tiles of one XCD touch when logical
// tiles run down `group` tile rows at a time (each XCD holds about cus_per_xcd tiles).
static int64_t xcd_panel_rows(int64_t tiles_m, int64_t tiles_n, int64_t group, int64_t bm, int64_t bn) {
    const int64_t cus_per_xcd = kNumCUs / 8;
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

struct GemmPlan {
    int tile, splits;
    int64_t tiles_m, tiles_n;
};

// Forced configuration for tuning and tests: a tile index (or -1 for the planner's
// choice) and a split count (or 0). Initialised from FP8Q_GEMM_TILE (a tile name) and
// FP8Q_GEMM_SPLITS, changed by gemm_force_config().
static std::atomic<int> g_forced_tile{-2}, g_forced_splits{-1};

static int env_tile() {
    int v = g_forced_tile.load(std::memory_order_relaxed);
    if (v == -2) {
        v = -1;
        if (const char *e = std::getenv("FP8Q_GEMM_TILE"))
            for (int t = 0; t < T_COUNT; ++t)
                if (std::strcmp(e, kTiles[t].name) == 0) v = t;
        int expected = -2;
        g_forced_tile.compare_exchange_strong(expected, v);
        v = g_forced_tile.load(std::memory_order_relaxed);
    }
    return v;
}
static int env_splits() {
    int v = g_forced_splits.load(std::memory_order_relaxed);
    if (v == -1) {
        const char *e = std::getenv("FP8Q_GEMM_SPLITS");
        const int n = e ? std::atoi(e) : 0;
        v = n >= 1 && n <= kMaxSplits ? n : 0;
        int expected = -1;
        g_forced_splits.compare_exchange_strong(expected, v);
        v = g_forced_splits.load(std::memory_order_relaxed);
    }
    return v;
}

bool gemm_force_config(int tile, int splits) {
    if (tile < -1 || tile >= T_COUNT || splits < 0 || splits > kMaxSplits) return false;
    g_forced_tile.store(tile, std::memory_order_relaxed);
    g_forced_splits.store(splits, std::memory_order_relaxed);
    return true;
}

const char *gemm_config_name(int tile) { return tile >= 0 && tile < T_COUNT ? kTiles[tile].name : nullptr; }

// Split-K workspace: the arrival words first, at a fixed place whatever the shape, then the
// partial tiles.
constexpr int64_t kMaxSplitTiles = 4096;
constexpr size_t kCounterBytes = kMaxSplitTiles * sizeof(uint64_t);

// Epoch of a split-K launch: never 0, so that a zero-filled workspace holds no arrivals of
// any launch. Launches that share a workspace run one after the other on one stream, so
// they only need different epochs, which a process-wide counter gives (until it wraps
// after 2^32 - 1 launches).
static std::atomic<uint32_t> g_epoch{0};
static uint32_t next_epoch() {
    uint32_t e;
    do e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    while (e == 0);
    return e;
}

static size_t split_bytes(const GemmPlan &p) {
    if (p.splits <= 1) return 0;
    const int64_t tiles = p.tiles_m * p.tiles_n;
    return kCounterBytes + (size_t)tiles * p.splits * kTiles[p.tile].bm * kTiles[p.tile].bn * sizeof(float);
}

// Estimated duration (us): full waves of workgroups times the slices each contracts plus
// its fixed cost, plus the split-K reduction (the last workgroup of a tile reads the other
// splits' partials; all of them write theirs).
static double plan_cost(int tile, int64_t tiles, int splits, int64_t nkb, bool exact) {
    const TileInfo &t = kTiles[tile];
    const double us_slice = exact && t.us_slice_x > 0 ? t.us_slice_x : t.us_slice;
    const double us_fixed = exact && t.us_slice_x > 0 ? t.us_fixed_x : t.us_fixed;
    const double kouts = t.bm * t.bn / 1024.0;
    const int64_t units = tiles * splits;
    const int64_t waves = (units + kNumCUs - 1) / kNumCUs;
    const double per_unit = (double)((nkb + splits - 1) / splits) * us_slice + us_fixed;
    return waves * per_unit + (splits - 1) * 0.23 * kouts;
}

static GemmPlan make_plan(int64_t M, int64_t N, int64_t K, bool exact, size_t ws_bytes, bool size_query,
                          bool rowb = false) {
    const int64_t nkb = K / G_SLICE;
    GemmPlan best{T128x128, 1, (M + 127) / 128, (N + 127) / 128};
    double best_cost = 1e300;
    const int forced_tile = env_tile(), forced_splits = exact ? 1 : env_splits();
    for (int t = 0; t < T_COUNT; ++t) {
        // a forced tile (tuning) is taken even where the planner would not pick it
        if (forced_tile >= 0 ? t != forced_tile : (exact ? !kTiles[t].exact_ok : !kTiles[t].fp8_ok)) continue;
        // (a forced tile without it leaves the default)
        if (rowb && !(kTiles[t].rowb_ok & (exact ? 2 : 1))) continue;
        const int64_t tm = (M + kTiles[t].bm - 1) / kTiles[t].bm, tn = (N + kTiles[t].bn - 1) / kTiles[t].bn;
        for (int s = 1; s <= (exact ? 1 : kMaxSplits); ++s) {
            // a split contracts at least 2 slices; a forced count falls back to 1 where it cannot apply
            if (s > 1 && (nkb < 2 * s || tm * tn > kMaxSplitTiles)) break;
            const GemmPlan p{t, s, tm, tn};
            if (s > 1 && !size_query && split_bytes(p) > ws_bytes) break;
            if (forced_splits && s != forced_splits && s != 1) continue;
            double c = plan_cost(t, tm * tn, s, nkb, exact);
            if (forced_splits && s == 1 && forced_splits != 1) c += 1e200;   // only if the forced count is impossible
            if (c < best_cost) {
                best_cost = c;
                best = p;
            }
        }
    }
    return best;
}

void gemm_plan(int64_t M, int64_t N, int64_t K, bool, bool exact, int *tile, int *splits) {
    const GemmPlan p = make_plan(M, N, K, exact, 0, true);
    // (what dispatch launches: a forced tile the exact-slice mode lacks runs as 128x128)
    *tile = exact && !kTiles[p.tile].exact_ok ? (int)T128x128 : p.tile;
    *splits = p.splits;
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool, bool exact, bool rowb) {
    return split_bytes(make_plan(M, N, K, exact, 0, true, rowb));
}

// Split-K scratch of launch_block_gemm_noalloc, for callers that cannot allocate: one array
// per GPU, allocated with the library's code object when it is loaded on that GPU and held
// until the process ends. Host code never passes `scratch` itself to a kernel (on the host it
// is only a stand-in for the symbol): the device address of each GPU's copy is looked up once
// per device with hipGetSymbolAddress and kept in g_scratch_addr.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kScratchDevices = 64;
static std::atomic<void *> g_scratch_addr[kScratchDevices];

// Device address of the current device's scratch (looked up on the device's first call).
static hipError_t current_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // racing first calls on one device look up the same address; either store is correct
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_block_gemm_noalloc(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, void *y,
                                     bool out_bf16, bool exact, bool sa_kmajor, int64_t M, int64_t N, int64_t K,
                                     hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    // the caller has checked that this shape's split-K plan fits the scratch; with that
    // capacity make_plan picks the same plan as launch_block_gemm given the full workspace
    if (gemm_workspace_bytes(M, N, K, out_bf16, exact) > kNoallocScratchBytes) return hipErrorInvalidValue;
    void *ws = nullptr;
    const hipError_t e = current_scratch(&ws);
    if (e != hipSuccess) return e;
    return launch_block_gemm(aq, sa, wq, sw, nullptr, y, out_bf16, exact, sa_kmajor, M, N, K, ws,
                             kNoallocScratchBytes, stream);
}

template <int BM, int BN, int NW, int WAVES_M, int NSTAGE, int EXACT, int GROUPED = 0, int ROWB = 0>
static hipError_t launch_cfg(GemmArgs a, bool out_bf16, int splits, hipStream_t stream) {
    // grouped: an upper bound on the m-tiles of all experts (sum of ceil(rows_e / BM))
    a.tiles_m = (int)((a.M + BM - 1) / BM + (a.offsets ? a.experts : 0));
    a.tiles_n = (int)((a.N + BN - 1) / BN);
    a.group = choose_group(a.tiles_m, a.tiles_n, BM, BN);
    a.splits = splits;
    // a grid dimension counts at most 2^32 - 1 work-items
    const int64_t units = (int64_t)a.tiles_m * a.tiles_n * splits;
    if (units * NW * 64 > 0xFFFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)units), block(NW * 64);
    if (out_bf16)
        block_gemm_kernel<BM, BN, NW, WAVES_M, NSTAGE, 1, EXACT, GROUPED, ROWB><<<grid, block, 0, stream>>>(a);
    else
        block_gemm_kernel<BM, BN, NW, WAVES_M, NSTAGE, 0, EXACT, GROUPED, ROWB><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

static hipError_t dispatch(const GemmPlan &p, const GemmArgs &a, bool out_bf16, bool exact, hipStream_t stream) {
    if (exact) {
        switch (p.tile) {
        case T256x256W8: return launch_cfg<256, 256, 8, 2, 2, 1>(a, out_bf16, 1, stream);
        case T256x128W8: return launch_cfg<256, 128, 8, 4, 3, 1>(a, out_bf16, 1, stream);
        case T128x256W8: return launch_cfg<128, 256, 8, 2, 3, 1>(a, out_bf16, 1, stream);
        case T128x192W8: return launch_cfg<128, 192, 8, 2, 3, 1>(a, out_bf16, 1, stream);
        default: return launch_cfg<128, 128, 4, 2, 4, 1>(a, out_bf16, 1, stream);
        }
    }
    switch (p.tile) {
    case T256x256W8: return launch_cfg<256, 256, 8, 2, 2, 0>(a, out_bf16, p.splits, stream);
    case T256x192W8: return launch_cfg<256, 192, 8, 2, 2, 0>(a, out_bf16, p.splits, stream);
    case T256x128W8: return launch_cfg<256, 128, 8, 4, 3, 0>(a, out_bf16, p.splits, stream);
    case T128x256W8: return launch_cfg<128, 256, 8, 2, 3, 0>(a, out_bf16, p.splits, stream);
    case T128x192W8: return launch_cfg<128, 192, 8, 2, 3, 0>(a, out_bf16, p.splits, stream);
    case T256x128: return launch_cfg<256, 128, 4, 2, 3, 0>(a, out_bf16, p.splits, stream);
    case T128x128S2: return launch_cfg<128, 128, 4, 2, 2, 0>(a, out_bf16, p.splits, stream);
    default: return launch_cfg<128, 128, 4, 2, 4, 0>(a, out_bf16, p.splits, stream);
    }
}

// per-row weight scales: the subset of tiles instantiated for them
static hipError_t dispatch_rowb(const GemmPlan &p, const GemmArgs &a, bool out_bf16, bool exact, hipStream_t stream) {
    if (exact) {
        switch (p.tile) {
        case T128x192W8: return launch_cfg<128, 192, 8, 2, 3, 1, 0, 1>(a, out_bf16, 1, stream);
        default: return launch_cfg<128, 128, 4, 2, 4, 1, 0, 1>(a, out_bf16, 1, stream);
        }
    }
    switch (p.tile) {
    case T256x128W8: return launch_cfg<256, 128, 8, 4, 3, 0, 0, 1>(a, out_bf16, p.splits, stream);
    case T128x256W8: return launch_cfg<128, 256, 8, 2, 3, 0, 0, 1>(a, out_bf16, p.splits, stream);
    case T128x192W8: return launch_cfg<128, 192, 8, 2, 3, 0, 0, 1>(a, out_bf16, p.splits, stream);
    default: return launch_cfg<128, 128, 4, 2, 4, 0, 0, 1>(a, out_bf16, p.splits, stream);
    }
}

hipError_t launch_rowwise_gemm(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb, void *y,
                               bool out_bf16, bool exact, int64_t M, int64_t N, int64_t K, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    const GemmPlan p = make_plan(M, N, K, exact, workspace ? workspace_bytes : 0, false, true);
    GemmArgs a{aq, sa, bq, sb, y, nullptr, nullptr, nullptr, 0, nullptr, M, N, K, 0, 0, 1, 1, 0, 0};
    if (p.splits > 1) {
        a.count = static_cast<uint64_t *>(workspace);
        a.epoch = next_epoch();
        a.part = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + kCounterBytes);
    }
    return dispatch_rowb(p, a, out_bf16, exact, stream);
}

hipError_t launch_block_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                             const float *bias, void *y, bool out_bf16, bool exact, bool sa_kmajor, int64_t M,
                             int64_t N, int64_t K, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (sa_kmajor && M * (K / G_SLICE) >= ((int64_t)1 << 29)) return hipErrorInvalidValue;
    const GemmPlan p = make_plan(M, N, K, exact, workspace ? workspace_bytes : 0, false);
    GemmArgs a{aq, sa, wq, sw, y, bias, nullptr, nullptr, 0, nullptr, M, N, K, 0, 0, 1, 1, 0, sa_kmajor ? 1 : 0};
    if (p.splits > 1) {
        a.count = static_cast<uint64_t *>(workspace);
        a.epoch = next_epoch();
        a.part = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + kCounterBytes);
    }
    return dispatch(p, a, out_bf16, exact, stream);
}

hipError_t launch_grouped_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                               const int64_t *offsets, void *y, bool out_bf16, bool exact, int64_t experts,
                               int64_t rows, int64_t N, int64_t K, hipStream_t stream) {
    if (rows == 0 || N == 0) return hipSuccess;
    // Few tiles are instantiated for the grouped kernel: BM = 128 keeps the padding of each
    // expert's last m-tile small; BN = 256 for wide weights, 192 otherwise.
    GemmArgs a{aq, sa, wq, sw, y, nullptr, nullptr, nullptr, 0, offsets, rows, N, K, 0, 0, 1, 1, (int)experts, 0};
    if (exact) return launch_cfg<128, 192, 8, 2, 3, 1, 1>(a, out_bf16, 1, stream);
    if (N >= 1024) return launch_cfg<128, 256, 8, 2, 3, 0, 1>(a, out_bf16, 1, stream);
    return launch_cfg<128, 192, 8, 2, 3, 0, 1>(a, out_bf16, 1, stream);
}

}  // namespace fp8q
