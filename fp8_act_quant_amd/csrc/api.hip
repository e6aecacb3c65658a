// api.hip -- the C ABI declared in include/fp8q.h: host-side validation, then one launch
// on the caller's stream. Nothing here allocates, synchronises or keeps state beyond a
// per-device "is this a gfx950" cache.
#include <fp8q.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "launch.h"

namespace {

constexpr int64_t kBlock = 128;
constexpr int kMaxDevices = 64;
// launch-geometry limits of the kernels (grid dimensions are 32-bit)
constexpr int64_t kMaxElems = (int64_t)1 << 46;
constexpr int64_t kMaxWeightBlockRows = 65535;
// The GEMM addresses a workgroup's rows of A and W (at most 256 rows of K bytes) through
// buffer resources whose byte count is 32-bit and which read zero past it: 256 * K must stay
// below 2^32, so K < 2^24 (a count of exactly 2^32 cannot be stated, and its last bytes would
// read as zero).
constexpr int64_t kMaxGemmK = ((int64_t)1 << 24) - 128;
// grid dimensions of the two-dimensional launches
constexpr int64_t kMaxGridX = 0x7FFFFFFF, kMaxGridY = 65535;
// a grid dimension counts at most 2^32 - 1 work-items: workgroups of 256 threads along it
constexpr int64_t kMaxBlocks256 = 0xFFFFFFFFll / 256;
// The bf16 GEMM advances K in steps of 64 elements and addresses a workgroup's rows (at most
// 256 of 2K bytes) through 32-bit buffer resources: K < 2^23.
constexpr int64_t kBf16Step = 64;
constexpr int64_t kMaxBf16K = ((int64_t)1 << 23) - kBf16Step;
// K-block-major activation scales are addressed with 32-bit byte offsets: M * K/128 < 2^29
constexpr int64_t kMaxKmajorScales = (int64_t)1 << 29;
// The GEMMs count tile rows and columns in 32-bit ints (64-row tiles at the smallest), and a
// grid holds at most 2^32 / 256 workgroups; with M, N <= 2^36 the counts stay far inside
// both. (No device holds such an operand: 2^36 rows of K >= 64 elements.)
constexpr int64_t kMaxGemmRows = (int64_t)1 << 36;

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// 0 = unknown, 1 = gfx950, 2 = other / unusable
std::atomic<int> g_dev_kind[kMaxDevices];

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FP8Q_ERR_UNSUPPORTED;
    if (dev < 0 || dev >= kMaxDevices) return FP8Q_ERR_UNSUPPORTED;
    int kind = g_dev_kind[dev].load(std::memory_order_relaxed);
    if (kind == 0) {
        hipDeviceProp_t prop;
        kind = 2;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
            kind = 1;
        g_dev_kind[dev].store(kind, std::memory_order_relaxed);
    }
    return kind == 1 ? FP8Q_OK : FP8Q_ERR_UNSUPPORTED;
}

int shape_ok(int64_t rows, int64_t K) {
    if (rows < 0 || K < 0 || (K % kBlock) != 0) return FP8Q_ERR_SHAPE;
    if (K > 0 && rows > kMaxElems / K) return FP8Q_ERR_SHAPE;
    return FP8Q_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_LAUNCH; }

}  // namespace

extern "C" {

int fp8_act_quant(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K, void *stream) {
    if (int e = shape_ok(M, K)) return e;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_ERR_NULL;
    if (misaligned(x, 16) || misaligned(q, 16) || misaligned(s, 4)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_act_quant(x, q, s, M, K, false, static_cast<hipStream_t>(stream)));
}

int fp8_act_quant_kmajor(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K, void *stream) {
    if (int e = shape_ok(M, K)) return e;
    if (K > 0 && M >= kMaxKmajorScales / (K / kBlock)) return FP8Q_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_ERR_NULL;
    if (misaligned(x, 16) || misaligned(q, 16) || misaligned(s, 4)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_act_quant(x, q, s, M, K, true, static_cast<hipStream_t>(stream)));
}

int fp8_weight_quant(const uint16_t *w, uint8_t *q, float *s, int64_t N, int64_t K, void *stream) {
    if (int e = shape_ok(N, K)) return e;
    if ((N + kBlock - 1) / kBlock > kMaxWeightBlockRows) return FP8Q_ERR_SHAPE;
    if (K / kBlock > kMaxBlocks256) return FP8Q_ERR_SHAPE;   // one workgroup per 128-column block
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!w || !q || !s) return FP8Q_ERR_NULL;
    if (misaligned(w, 16) || misaligned(q, 16) || misaligned(s, 4)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_weight_quant(w, q, s, N, K, static_cast<hipStream_t>(stream)));
}

int fp8_weight_dequant(const uint8_t *q, const float *s, uint16_t *w, int64_t N, int64_t K, void *stream) {
    if (int e = shape_ok(N, K)) return e;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!w || !q || !s) return FP8Q_ERR_NULL;
    if (misaligned(w, 16) || misaligned(q, 16) || misaligned(s, 4)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_weight_dequant(q, s, w, N, K, static_cast<hipStream_t>(stream)));
}

int fp8_block_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, void *y,
                   int y_dtype, int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                   void *stream) {
    return fp8_block_gemm_bias(aq, sa, wq, sw, nullptr, y, y_dtype, M, N, K, workspace, workspace_bytes, stream);
}

int fp8_block_gemm_bias(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, const float *bias,
                        void *y, int y_dtype, int64_t M, int64_t N, int64_t K, void *workspace,
                        size_t workspace_bytes, void *stream) {
    const int dtype = y_dtype & 0xFF;
    const bool sa_kmajor = (y_dtype & FP8Q_SA_KMAJOR) != 0;
    const int mode = y_dtype & ~0xFF & ~FP8Q_SA_KMAJOR;
    if (dtype != FP8Q_OUT_F32 && dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
    if (mode != 0 && mode != FP8Q_GEMM_FP8_PRODUCTS && mode != FP8Q_GEMM_EXACT_SLICES) return FP8Q_ERR_DTYPE;
    if (int e = shape_ok(M, K)) return e;
    if (int e = shape_ok(N, K)) return e;
    if (M > 0 && N > kMaxElems / M) return FP8Q_ERR_SHAPE;
    if (K > kMaxGemmK || M > kMaxGemmRows || N > kMaxGemmRows) return FP8Q_ERR_SHAPE;
    if (sa_kmajor && K > 0 && M >= kMaxKmajorScales / (K / kBlock)) return FP8Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!y) return FP8Q_ERR_NULL;
    if (K > 0 && (!aq || !sa || !wq || !sw)) return FP8Q_ERR_NULL;
    if (misaligned(aq, 16) || misaligned(wq, 16) || misaligned(y, 16) || misaligned(sa, 4) ||
        misaligned(sw, 4) || misaligned(bias, 4))
        return FP8Q_ERR_ALIGN;
    if (workspace == nullptr) workspace_bytes = 0;
    if (workspace_bytes && misaligned(workspace, 16)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    // default contraction: exact slices for fp32 output, the FP8 matrix unit for bf16 output
    const bool exact = mode == FP8Q_GEMM_EXACT_SLICES || (mode == 0 && dtype == FP8Q_OUT_F32);
    return finish(fp8q::launch_block_gemm(aq, sa, wq, sw, bias, y, dtype == FP8Q_OUT_BF16, exact, sa_kmajor, M, N,
                                          K, workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

int fp8_bf16_gemm(const uint16_t *x, const uint16_t *w, const float *bias, void *y, int y_dtype, int64_t M,
                  int64_t N, int64_t K, void *stream) {
    if (y_dtype != FP8Q_OUT_F32 && y_dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || (K % kBf16Step) != 0 || K > kMaxBf16K) return FP8Q_ERR_SHAPE;
    if ((K > 0 && (M > kMaxElems / K || N > kMaxElems / K)) || (M > 0 && N > kMaxElems / M)) return FP8Q_ERR_SHAPE;
    if (M > kMaxGemmRows || N > kMaxGemmRows) return FP8Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!y || (K > 0 && (!x || !w))) return FP8Q_ERR_NULL;
    if (misaligned(x, 16) || misaligned(w, 16) || misaligned(y, 4) || misaligned(bias, 4)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_bf16_gemm(x, w, bias, y, y_dtype == FP8Q_OUT_BF16, M, N, K,
                                         static_cast<hipStream_t>(stream)));
}

int fp8_block_gemm_noalloc(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, void *y,
                           int y_dtype, int64_t M, int64_t N, int64_t K, void *stream) {
    static_assert(FP8Q_NOALLOC_SCRATCH_BYTES == fp8q::kNoallocScratchBytes, "scratch size in the header");
    const int dtype = y_dtype & 0xFF;
    const bool sa_kmajor = (y_dtype & FP8Q_SA_KMAJOR) != 0;
    const int mode = y_dtype & ~0xFF & ~FP8Q_SA_KMAJOR;
    if (dtype != FP8Q_OUT_F32 && dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
    if (mode != 0 && mode != FP8Q_GEMM_FP8_PRODUCTS && mode != FP8Q_GEMM_EXACT_SLICES) return FP8Q_ERR_DTYPE;
    if (int e = shape_ok(M, K)) return e;
    if (int e = shape_ok(N, K)) return e;
    if (M > 0 && N > kMaxElems / M) return FP8Q_ERR_SHAPE;
    if (K > kMaxGemmK || M > kMaxGemmRows || N > kMaxGemmRows) return FP8Q_ERR_SHAPE;
    if (sa_kmajor && K > 0 && M >= kMaxKmajorScales / (K / kBlock)) return FP8Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8Q_OK;
    const bool exact = mode == FP8Q_GEMM_EXACT_SLICES || (mode == 0 && dtype == FP8Q_OUT_F32);
    // the split-K plan fp8_block_gemm would use with its full workspace must fit the static scratch
    if (K > 0 && fp8q::gemm_workspace_bytes(M, N, K, dtype == FP8Q_OUT_BF16, exact) > FP8Q_NOALLOC_SCRATCH_BYTES)
        return FP8Q_ERR_WORKSPACE;
    if (!y) return FP8Q_ERR_NULL;
    if (K > 0 && (!aq || !sa || !wq || !sw)) return FP8Q_ERR_NULL;
    if (misaligned(aq, 16) || misaligned(wq, 16) || misaligned(y, 16) || misaligned(sa, 4) || misaligned(sw, 4))
        return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_block_gemm_noalloc(aq, sa, wq, sw, y, dtype == FP8Q_OUT_BF16, exact, sa_kmajor, M, N,
                                                  K, static_cast<hipStream_t>(stream)));
}

int fp8_grouped_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, const int64_t *offsets,
                     void *y, int y_dtype, int64_t experts, int64_t rows, int64_t N, int64_t K, void *stream) {
    const int dtype = y_dtype & 0xFF;
    const int mode = y_dtype & ~0xFF;
    if (dtype != FP8Q_OUT_F32 && dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
    if (mode != 0 && mode != FP8Q_GEMM_FP8_PRODUCTS && mode != FP8Q_GEMM_EXACT_SLICES) return FP8Q_ERR_DTYPE;
    if (experts < 1 || experts > fp8q::kMaxGroupedExperts) return FP8Q_ERR_SHAPE;
    if (int e = shape_ok(rows, K)) return e;
    if (int e = shape_ok(N, K)) return e;
    if (N > 0 && experts > kMaxElems / N) return FP8Q_ERR_SHAPE;
    if (int e = shape_ok(experts * N, K)) return e;
    if (rows > 0 && N > kMaxElems / rows) return FP8Q_ERR_SHAPE;
    if (K > kMaxGemmK || rows > INT32_MAX / 2 || N > kMaxGemmRows) return FP8Q_ERR_SHAPE;
    if (rows == 0 || N == 0) return FP8Q_OK;
    if (!y || !offsets) return FP8Q_ERR_NULL;
    if (K > 0 && (!aq || !sa || !wq || !sw)) return FP8Q_ERR_NULL;
    if (misaligned(aq, 16) || misaligned(wq, 16) || misaligned(y, 16) || misaligned(sa, 4) || misaligned(sw, 4) ||
        misaligned(offsets, 8))
        return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    const bool exact = mode == FP8Q_GEMM_EXACT_SLICES || (mode == 0 && dtype == FP8Q_OUT_F32);
    return finish(fp8q::launch_grouped_gemm(aq, sa, wq, sw, offsets, y, dtype == FP8Q_OUT_BF16, exact, experts, rows,
                                            N, K, static_cast<hipStream_t>(stream)));
}

int fp8_act_quant_t(const uint16_t *x, uint8_t *qt, float *st, int64_t M, int64_t C, void *stream) {
    if (M < 0 || C < 0 || (C % 8) != 0) return FP8Q_ERR_SHAPE;
    const int64_t ldq = (M + kBlock - 1) / kBlock * kBlock;
    if ((C > 0 && ldq > kMaxElems / C) || (C + 127) / 128 > kMaxGridY || ldq / kBlock > kMaxBlocks256) return FP8Q_ERR_SHAPE;
    if (M == 0 || C == 0) return FP8Q_OK;
    if (!x || !qt || !st) return FP8Q_ERR_NULL;
    if (misaligned(x, 16) || misaligned(qt, 16) || misaligned(st, 4)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_act_quant_t(x, qt, st, M, C, static_cast<hipStream_t>(stream)));
}

int fp8_weight_transpose(const uint8_t *wq, const float *sw, uint8_t *wqt, float *swt, int64_t N, int64_t K,
                         void *stream) {
    if (int e = shape_ok(N, K)) return e;
    if ((N + 63) / 64 > kMaxGridY || K / 64 > kMaxBlocks256) return FP8Q_ERR_SHAPE;   // 64x64-byte tiles
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!wq || !sw || !wqt || !swt) return FP8Q_ERR_NULL;
    if (misaligned(wq, 16) || misaligned(wqt, 16) || misaligned(sw, 4) || misaligned(swt, 4)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    return finish(fp8q::launch_weight_transpose(wq, sw, wqt, swt, N, K, static_cast<hipStream_t>(stream)));
}

int fp8_rowwise_gemm(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb, void *y, int y_dtype,
                     int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
    const int dtype = y_dtype & 0xFF;
    const int mode = y_dtype & ~0xFF;
    if (dtype != FP8Q_OUT_F32 && dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
    if (mode != 0 && mode != FP8Q_GEMM_FP8_PRODUCTS && mode != FP8Q_GEMM_EXACT_SLICES) return FP8Q_ERR_DTYPE;
    if (int e = shape_ok(M, K)) return e;
    if (int e = shape_ok(N, K)) return e;
    if (M > 0 && N > kMaxElems / M) return FP8Q_ERR_SHAPE;
    if (K > kMaxGemmK || M > kMaxGemmRows || N > kMaxGemmRows) return FP8Q_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!y) return FP8Q_ERR_NULL;
    if (K > 0 && (!aq || !sa || !bq || !sb)) return FP8Q_ERR_NULL;
    if (misaligned(aq, 16) || misaligned(bq, 16) || misaligned(y, 16) || misaligned(sa, 4) || misaligned(sb, 4))
        return FP8Q_ERR_ALIGN;
    if (workspace == nullptr) workspace_bytes = 0;
    if (workspace_bytes && misaligned(workspace, 16)) return FP8Q_ERR_ALIGN;
    if (int e = check_device()) return e;
    const bool exact = mode == FP8Q_GEMM_EXACT_SLICES || (mode == 0 && dtype == FP8Q_OUT_F32);
    return finish(fp8q::launch_rowwise_gemm(aq, sa, bq, sb, y, dtype == FP8Q_OUT_BF16, exact, M, N, K, workspace,
                                            workspace_bytes, static_cast<hipStream_t>(stream)));
}

size_t fp8_rowwise_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int y_dtype) {
    if (M <= 0 || N <= 0 || K <= 0 || (K % kBlock) != 0 || K > kMaxGemmK) return 0;
    if (N > kMaxElems / M || shape_ok(M, K) || shape_ok(N, K) || M > kMaxGemmRows || N > kMaxGemmRows) return 0;
    const int dtype = y_dtype & 0xFF;
    const int mode = y_dtype & ~0xFF;
    if (dtype != FP8Q_OUT_F32 && dtype != FP8Q_OUT_BF16) return 0;
    if (mode != 0 && mode != FP8Q_GEMM_FP8_PRODUCTS && mode != FP8Q_GEMM_EXACT_SLICES) return 0;
    const bool exact = mode == FP8Q_GEMM_EXACT_SLICES || (mode == 0 && dtype == FP8Q_OUT_F32);
    return fp8q::gemm_workspace_bytes(M, N, K, dtype == FP8Q_OUT_BF16, exact, true);
}

size_t fp8_block_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int y_dtype) {
    if (M <= 0 || N <= 0 || K <= 0 || (K % kBlock) != 0 || K > kMaxGemmK) return 0;
    if (N > kMaxElems / M || shape_ok(M, K) || shape_ok(N, K) || M > kMaxGemmRows || N > kMaxGemmRows) return 0;
    const int dtype = y_dtype & 0xFF;
    const int mode = y_dtype & ~0xFF & ~FP8Q_SA_KMAJOR;   // (the scale layout does not change the plan)
    if (dtype != FP8Q_OUT_F32 && dtype != FP8Q_OUT_BF16) return 0;
    if (mode != 0 && mode != FP8Q_GEMM_FP8_PRODUCTS && mode != FP8Q_GEMM_EXACT_SLICES) return 0;
    const bool exact = mode == FP8Q_GEMM_EXACT_SLICES || (mode == 0 && dtype == FP8Q_OUT_F32);
    return fp8q::gemm_workspace_bytes(M, N, K, dtype == FP8Q_OUT_BF16, exact);
}

int fp8q_gemm_force_config(int config, int splits) {
    return fp8q::gemm_force_config(config, splits) ? FP8Q_OK : FP8Q_ERR_SHAPE;
}

const char *fp8q_gemm_config_name(int config) { return fp8q::gemm_config_name(config); }

int fp8q_gemm_plan(int64_t M, int64_t N, int64_t K, int y_dtype, int *config, int *splits) {
    if (!config || !splits) return FP8Q_ERR_NULL;
    const int dtype = y_dtype & 0xFF;
    const int mode = y_dtype & ~0xFF & ~FP8Q_SA_KMAJOR;   // (the scale layout does not change the plan)
    if (dtype != FP8Q_OUT_F32 && dtype != FP8Q_OUT_BF16) return FP8Q_ERR_DTYPE;
    if (mode != 0 && mode != FP8Q_GEMM_FP8_PRODUCTS && mode != FP8Q_GEMM_EXACT_SLICES) return FP8Q_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || (K % kBlock) != 0 || K > kMaxGemmK) return FP8Q_ERR_SHAPE;
    if (N > kMaxElems / M || shape_ok(M, K) || shape_ok(N, K) || M > kMaxGemmRows || N > kMaxGemmRows)
        return FP8Q_ERR_SHAPE;
    const bool exact = mode == FP8Q_GEMM_EXACT_SLICES || (mode == 0 && dtype == FP8Q_OUT_F32);
    fp8q::gemm_plan(M, N, K, dtype == FP8Q_OUT_BF16, exact, config, splits);
    return FP8Q_OK;
}

const char *fp8q_strerror(int status) {
    switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_ERR_NULL: return "a required pointer is NULL";
    case FP8Q_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of 128, or too large)";
    case FP8Q_ERR_ALIGN: return "pointer alignment below what the entry point requires";
    case FP8Q_ERR_DTYPE: return "unknown output dtype";
    case FP8Q_ERR_UNSUPPORTED: return "no gfx950 device is current";
    case FP8Q_ERR_LAUNCH: return "kernel launch failed";
    case FP8Q_ERR_WORKSPACE:
        return "the shape's split-K schedule needs more scratch than the static scratch holds "
               "(FP8Q_NOALLOC_SCRATCH_BYTES); call fp8_block_gemm with a workspace instead";
    default: return "unknown status";
    }
}

int fp8q_version(void) { return (1 << 16) | 5; }

}  // extern "C"
