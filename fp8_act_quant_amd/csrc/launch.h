// launch.h -- internal host-side launchers behind the C ABI (include/fp8q.h).
// They assume validated arguments and enqueue on `stream`; they return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8q {

// kmajor: scales written K-block-major, s[kb * M + m] (M * K/128 < 2^32), else s[m * K/128 + kb]
hipError_t launch_act_quant(const uint16_t *x, uint8_t *q, float *s, int64_t M, int64_t K, bool kmajor,
                            hipStream_t stream);
hipError_t launch_weight_quant(const uint16_t *w, uint8_t *q, float *s, int64_t N, int64_t K,
                               hipStream_t stream);
hipError_t launch_weight_dequant(const uint8_t *q, const float *s, uint16_t *w, int64_t N, int64_t K,
                                 hipStream_t stream);

// Block-scaled GEMM. out_bf16 selects the output dtype; exact selects the exact-slice
// contraction (f16 matrix unit on exactly converted operands) instead of the FP8 matrix
// unit. bias (fp32 [N], may be NULL) is added in fp32 before the output rounding. The
// workspace (may be NULL, any contents) is used for a split-K schedule when workspace_bytes >=
// gemm_workspace_bytes(M, N, K, out_bf16, exact).
// sa_kmajor: sa is K-block-major [K/128, M] (M * K/128 < 2^29), else row-major [M, K/128].
hipError_t launch_block_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                             const float *bias, void *y, bool out_bf16, bool exact, bool sa_kmajor, int64_t M,
                             int64_t N, int64_t K, void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool out_bf16, bool exact, bool rowb = false);

// launch_block_gemm (no bias) with the library's static per-GPU split-K scratch of
// kNoallocScratchBytes instead of a caller's workspace; allocates nothing. The shape's
// gemm_workspace_bytes must not exceed kNoallocScratchBytes (hipErrorInvalidValue otherwise).
// Calls on one GPU share that scratch, so calls that overlap on one GPU race.
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t launch_block_gemm_noalloc(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw, void *y,
                                     bool out_bf16, bool exact, bool sa_kmajor, int64_t M, int64_t N, int64_t K,
                                     hipStream_t stream);

// Y = X . W^T on bf16 operands (the bf16 branch of linear()): x [M, K], w [N, K] bf16
// bits, fp32 accumulation, optional fp32 bias [N], Y fp32 or bf16 (RNE). K a multiple of 64
// below 2^23.
hipError_t launch_bf16_gemm(const uint16_t *x, const uint16_t *w, const float *bias, void *y, bool out_bf16, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream);

// GEMM with per-row scales on both operands: Y = sum over slices kb of
// (sum_k aq[m,k] bq[n,k]) * sa[m,kb] * sb[n,kb], sb [N, K/128]. Otherwise as launch_block_gemm
// (no bias); its workspace size is gemm_workspace_bytes(..., rowb = true).
hipError_t launch_rowwise_gemm(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb, void *y,
                               bool out_bf16, bool exact, int64_t M, int64_t N, int64_t K, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

// Training-side layout kernels. act_quant_t: x [M, C] bf16 -> qt [C, ldq] E4M3 and
// st [C, ldq / 128], ldq = ceil(M / 128) * 128: the 1x128 tiles run along the token
// dimension (column tiles of x), tokens past M are zero. weight_transpose: wq [N, K] ->
// wqt [K, N], sw [ceil(N/128), K/128] -> swt [K/128, ceil(N/128)].
hipError_t launch_act_quant_t(const uint16_t *x, uint8_t *qt, float *st, int64_t M, int64_t C, hipStream_t stream);
hipError_t launch_weight_transpose(const uint8_t *wq, const float *sw, uint8_t *wqt, float *swt, int64_t N,
                                   int64_t K, hipStream_t stream);

// Grouped GEMM over `experts` weight matrices: expert e multiplies rows [offsets[e],
// offsets[e+1]) of A (device int64 offsets, clamped to [0, rows]) by wq + e*N*K.
constexpr int64_t kMaxGroupedExperts = 1024;
hipError_t launch_grouped_gemm(const uint8_t *aq, const float *sa, const uint8_t *wq, const float *sw,
                               const int64_t *offsets, void *y, bool out_bf16, bool exact, int64_t experts,
                               int64_t rows, int64_t N, int64_t K, hipStream_t stream);
// tuning / test hook: force a tile configuration (-1: planner) and split count (0: planner)
bool gemm_force_config(int tile, int splits);
const char *gemm_config_name(int tile);
// the tile configuration and split count launch_block_gemm picks for a shape, given a
// workspace of at least gemm_workspace_bytes
void gemm_plan(int64_t M, int64_t N, int64_t K, bool out_bf16, bool exact, int *tile, int *splits);

}  // namespace fp8q
