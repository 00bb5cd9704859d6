// ss_mfma.h -- bf16 matrix-core helpers for the SSD kernels (gfx950).
//
// Operand layouts of the two products used, for lane l of a wavefront
// (li = l % 16, lg = l / 16), as measured on gfx950:
//   16x16x16 bf16: A[li][4 lg + e], B[4 lg + e][li], e = 0..3
//   16x16x32 bf16: A[li][8 lg + e], B[8 lg + e][li], e = 0..7
//   result (both): D[4 lg + r][li], r = 0..3
// So a result tile X, its four values per lane rounded to bf16, is the B
// operand of a 16x16x16 product as it stands, and the A operand for X^T.
#pragma once

#include "ss_device.h"

namespace ssk {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8_t a, bf16x8_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short bfs(float v) { return static_cast<short>(f32_to_bf16(v)); }

// v = hi + lo with hi = bfs(v) and lo = lo_bf(v, hi): the part of v that
// one bf16 misses, in a second bf16
__device__ __forceinline__ short lo_bf(float v, short hi) {
    return bfs(v - bf16_to_f32(static_cast<bf16_t>(hi)));
}

// the four values of a result tile as bf16 high and low parts
__device__ __forceinline__ void split4(const f32x4 &v, s16x4 &hi, s16x4 &lo) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const short h = bfs(v[r]);
        hi[r] = h;
        lo[r] = lo_bf(v[r], h);
    }
}

// three bf16 parts, v = hi + mid + lo to about 2^-27 relative
__device__ __forceinline__ void split4x3(const f32x4 &v, s16x4 &hi, s16x4 &mid, s16x4 &lo) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const short h = bfs(v[r]);
        const float r1 = v[r] - bf16_to_f32(static_cast<bf16_t>(h));
        const short m = bfs(r1);
        hi[r] = h;
        mid[r] = m;
        lo[r] = bfs(r1 - bf16_to_f32(static_cast<bf16_t>(m)));
    }
}

// two 4-value halves as one 8-value operand (elements copied by value:
// clang takes the bit cast of a vector element from element 0)
__device__ __forceinline__ bf16x8_t cat8(const s16x4 &a, const s16x4 &b) {
    bf16x8_t r;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const short x = a[e], y = b[e];
        r[e] = __builtin_bit_cast(__bf16, x);
        r[4 + e] = __builtin_bit_cast(__bf16, y);
    }
    return r;
}

constexpr f32x4 kZero4 = {0.0f, 0.0f, 0.0f, 0.0f};

// Inclusive running sum of a over the 64 lanes of a wavefront as an
// unevaluated pair hi + lo (compensated with the error-free two-sum of
// Knuth and Moller).  Decays exp(cum_t - cum_s) are then taken from
// (hi_t - hi_s) + (lo_t - lo_s): a plain f32 running sum would lose the
// low digits of a difference once the sum has grown large.
__device__ __forceinline__ void running_sum2(float a, int lane, float &hi, float &lo) {
    hi = a;
    lo = 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float oh = __shfl_up(hi, off, 64), ol = __shfl_up(lo, off, 64);
        if (lane >= off) {
            const float s = hi + oh, bb = s - hi;
            const float e = (hi - (s - bb)) + (oh - bb);
            const float l = lo + ol + e;
            hi = s + l;
            lo = l - (hi - s);
        }
    }
}

}  // namespace ssk
