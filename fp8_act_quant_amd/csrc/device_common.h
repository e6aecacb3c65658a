// device_common.h -- gfx950 device helpers shared by the quantisation and GEMM kernels.
//
// E4M3 here is OCP E4M3FN (bias 7, largest finite 448, no infinities), the format gfx950's
// v_cvt_pk_fp8_f32 / v_cvt_pk_f32_fp8 and the f8f6f4 MFMA (format code 0) implement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;            // quantisation granule along K (and along N for W)
constexpr float kE4M3Max = 448.0f;     // largest finite E4M3FN value

// Division by a per-tile scale d is done as y = RN(1/d) once per tile, then per element
//   q0 = RN(x * y);  r = x - q0 * d (exact, by FMA);  q = RN(q0 + r * y)   (Markstein).
// Over every (x, amax) pair of bf16 values this equals the IEEE quotient RN(x / d)
// wherever the quotient is >= 2^-11, and with the sign taken from x it gives the same
// E4M3 code as RN(x / d) for every pair (both checked exhaustively; below 2^-11 every
// result encodes to a signed zero). It needs d >= 2^-92 so that the
// residual cannot underflow; tiles with smaller scales take the IEEE division.
constexpr float kFastDivMin = 0x1p-92f;

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// max of the bf16 magnitudes (bit patterns with the sign cleared; for non-NaN bf16
// the unsigned order of these patterns is the order of |x|) held in one 32-bit word.
__device__ __forceinline__ uint32_t absmax_bits2(uint32_t w) {
    uint32_t a = w & 0x7FFF7FFFu;
    uint32_t lo = a & 0xFFFFu, hi = a >> 16;
    return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t absmax_bits8(u32x4 v) {
    uint32_t m0 = absmax_bits2(v.x), m1 = absmax_bits2(v.y);
    uint32_t m2 = absmax_bits2(v.z), m3 = absmax_bits2(v.w);
    m0 = m0 > m1 ? m0 : m1;
    m2 = m2 > m3 ? m2 : m3;
    return m0 > m2 ? m0 : m2;
}

// unsigned max across each aligned group of 16 lanes (one DPP row): after the two quad
// permutations every lane holds its quad's max, the half-row mirror pairs quads 0/1 and
// 2/3, and the row mirror pairs the two halves.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false); // row_half_mirror
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false); // row_mirror
    v = v > t ? v : t;
    return v;
}

// Per-tile constants: scale s = RN(amax / 448) (IEEE division), divisor d (1 for an
// all-zero tile), its correctly rounded reciprocal and whether the fast division applies.
struct TileScale {
    float s, d, y;
    bool fast;
};

__device__ __forceinline__ TileScale tile_scale(uint32_t amax_bits) {
    TileScale t;
    float amax = __uint_as_float(amax_bits << 16);
    t.s = amax / kE4M3Max;
    t.d = (amax_bits == 0) ? 1.0f : t.s;
    t.y = 1.0f / t.d;
    t.fast = t.d >= kFastDivMin;
    return t;
}

// The sign is taken from x: the quotient's sign is x's, and the correction step alone
// would turn a -0 (or a tiny negative quotient that cancels) into +0.
__device__ __forceinline__ float fast_quotient(float x, const TileScale &t) {
    float q0 = x * t.y;
    float r = __builtin_fmaf(-q0, t.d, x);
    return __builtin_copysignf(__builtin_fmaf(r, t.y, q0), x);
}

// E4M3 codes of 8 bf16 values (one 16-byte chunk) divided by the tile scale; returned as
// 8 bytes, element i in byte i. Saturation: the quotient is clamped to [-448, 448]
// before the round-to-nearest-even conversion.
__device__ __forceinline__ u32x2 quant8(u32x4 v, const TileScale &t) {
    float x[8] = {bf16lo_to_f32(v.x), bf16hi_to_f32(v.x), bf16lo_to_f32(v.y), bf16hi_to_f32(v.y),
                  bf16lo_to_f32(v.z), bf16hi_to_f32(v.z), bf16lo_to_f32(v.w), bf16hi_to_f32(v.w)};
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = fast_quotient(x[i], t);
    if (!t.fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = x[i] / t.d;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(q[i], -kE4M3Max, kE4M3Max);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
    return u32x2{(uint32_t)lo, (uint32_t)hi};
}

// fp32 pair -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t f = {a, b};
    bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

}  // namespace fp8q
