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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// Two values rounded to nearest-even bf16 by one instruction
// (v_cvt_pk_bf16_f32), a in the low half: the same bits as two bfs calls.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2_t r = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

// The hi / lo split of two values, each half packed as pk_bf16 packs it.
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pk_bf16(a, b);
    lo = pk_bf16(a - bf_lo(hi), b - bf_hi(hi));
}

__device__ __forceinline__ s16x4 s16x4_of(uint32_t w0, uint32_t w1) {
    return __builtin_bit_cast(s16x4, (u32x2_t){w0, w1});
}
__device__ __forceinline__ bf16x8_t bf16x8_of(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    return __builtin_bit_cast(bf16x8_t, (u32x4_t){w0, w1, w2, w3});
}

// the four values of a result tile as bf16 high and low parts
__device__ __forceinline__ void split4(const f32x4 &v, s16x4 &hi, s16x4 &lo) {
    uint32_t h0, l0, h1, l1;
    split2(v[0], v[1], h0, l0);
    split2(v[2], v[3], h1, l1);
    hi = s16x4_of(h0, h1);
    lo = s16x4_of(l0, l1);
}

// three bf16 parts, v = hi + mid + lo to about 2^-27 relative
__device__ __forceinline__ void split4x3(const f32x4 &v, s16x4 &hi, s16x4 &mid, s16x4 &lo) {
    uint32_t h[2], m[2], l[2];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const float a = v[2 * k], b = v[2 * k + 1];
        h[k] = pk_bf16(a, b);
        const float ra = a - bf_lo(h[k]), rb = b - bf_hi(h[k]);
        m[k] = pk_bf16(ra, rb);
        l[k] = pk_bf16(ra - bf_lo(m[k]), rb - bf_hi(m[k]));
    }
    hi = s16x4_of(h[0], h[1]);
    mid = s16x4_of(m[0], m[1]);
    lo = s16x4_of(l[0], l[1]);
}

// two 4-value halves as one 8-value operand (whole vectors: clang takes the
// bit cast of a single vector element from element 0)
__device__ __forceinline__ bf16x8_t cat8(const s16x4 &a, const s16x4 &b) {
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

constexpr f32x4 kZero4 = {0.0f, 0.0f, 0.0f, 0.0f};

// Inclusive running sum of a over the 64 lanes of a wavefront as an
// unevaluated pair hi + lo (compensated with the error-free two-sum of
// Knuth and Moller).  Decays exp(cum_t - cum_s) are then taken from
// (hi_t - hi_s) + (lo_t - lo_s): a plain f32 running sum would lose the
// low digits of a difference once the sum has grown large.  The partial
// sums move by DPP: shifts by 1, 2, 4 and 8 within each row of 16 lanes,
// then the last lane of rows 0 and 2 into rows 1 and 3, then lane 31 into
// rows 2 and 3; each step adds the pair it receives with the two-sum.
template <int CTRL, int ROWS>
__device__ __forceinline__ void running_sum2_step(float &hi, float &lo, bool take) {
    const float oh = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(hi), CTRL, ROWS, 0xf, false));
    const float ol = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(lo), CTRL, ROWS, 0xf, false));
    if (take) {
        const float s = hi + oh, bb = s - hi;
        const float e = (hi - (s - bb)) + (oh - bb);
        const float l = lo + ol + e;
        hi = s + l;
        lo = l - (hi - s);
    }
}
__device__ __forceinline__ void running_sum2(float a, int lane, float &hi, float &lo) {
    hi = a;
    lo = 0.0f;
    const int lr = lane & 15, row = lane >> 4;
    running_sum2_step<0x111, 0xf>(hi, lo, lr >= 1);   // row_shr:1
    running_sum2_step<0x112, 0xf>(hi, lo, lr >= 2);
    running_sum2_step<0x114, 0xf>(hi, lo, lr >= 4);
    running_sum2_step<0x118, 0xf>(hi, lo, lr >= 8);
    running_sum2_step<0x142, 0xa>(hi, lo, row & 1);     // row_bcast:15 into rows 1, 3
    running_sum2_step<0x143, 0xc>(hi, lo, row >= 2);    // row_bcast:31 into rows 2, 3
}

}  // namespace ssk
