// ss_device.h -- device helpers of the gfx950 selective-scan kernels.
//
// bf16 <-> f32 conversion, the f32 transcendental building blocks of the
// scan (exp2 on the hardware's v_exp_f32, softplus, sigmoid), and the DPP
// row broadcast used to share per-time-step scalars across the 16 lanes
// that hold one channel's 16 state entries.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssk {

// d_state handled by the kernels: one lane per state entry, 16 lanes per
// (batch, channel) row -- one DPP row of a 64-wide wavefront.
constexpr int kN = 16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint16_t bf16_t;  // bfloat16 carried as raw bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest-even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(bf16_t, h);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// 2^x on the hardware exponential unit.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(x) = log(1 + e^x) in f32.  For x > 20 the result equals x to
// within e^-20 relative.  Otherwise log1p(e) with e = e^x is log(w) plus the
// rounding error of w = 1 + e: d = e - (w - 1) is exact, and
// log(w + d) = log(w) + d / w + O(d^2).  d matters only while e is small
// (w < 2), where 1 / w = 2 - w + O(e^2); beyond, d / w is below half an ulp
// of the result and the term is dropped.  This keeps the result accurate to
// a few ulp even when e is tiny (w == 1 gives e), with one transcendental
// fewer than dividing by w - 1.
__device__ __forceinline__ float softplus_f32(float x) {
    float e = exp2_hw(x * kLog2e);
    float w = 1.0f + e;
    float d = e - (w - 1.0f);
    float lg = __builtin_amdgcn_logf(w) * kLn2;  // v_log_f32 is log2
    float r = __builtin_fmaf(d, __builtin_fmaxf(2.0f - w, 0.0f), lg);
    return x > 20.0f ? x : r;
}

// sigmoid(x) = 1 / (1 + e^-x); saturates cleanly to 0 and 1.
__device__ __forceinline__ float sigmoid_f32(float x) {
    return __builtin_amdgcn_rcpf(1.0f + exp2_hw(-x * kLog2e));
}

// Broadcast lane LANE of each 16-lane DPP row to the whole row
// (row_newbcast; one VALU op, or folded into the consuming instruction).
// The source lane always exists, so no "old" value is needed (bound_ctrl
// set lets the compiler fold the broadcast into a VOP2 consumer).
template <int LANE>
__device__ __forceinline__ float row_bcast(float v) {
    static_assert(LANE >= 0 && LANE < 16, "lane within a DPP row");
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + LANE, 0xf, 0xf, true));
}

// acc + (lane LANE of x's DPP row) * y as a single v_fmac_f32 with a row
// broadcast on x; the compiler folds broadcasts into multiplies and adds but
// not into fmac.  A DPP read of a VGPR needs two wait states after the VALU
// op that wrote it; the s_nop in the same asm block provides them whatever
// instruction the compiler scheduled in front.  NOP = false leaves it out, for
// a chain's later steps whose broadcast source was written long before (the
// build's assembly is checked for such reads).
// The lane is spelled into the asm text: an immediate operand would make
// the compiler treat the statement as a possible memory access and keep LDS
// loads from moving across it.
template <int LANE, bool NOP = true>
__device__ __forceinline__ float fmac_bcast(float acc, float x, float y) {
    static_assert(LANE >= 0 && LANE < 16, "lane within a DPP row");
    switch (LANE) {
#define SS_FMAC_BCAST(L)                                                                        \
    case L:                                                                                     \
        if constexpr (NOP)                                                                      \
            __asm__("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:" #L                    \
                    " row_mask:0xf bank_mask:0xf"                                               \
                    : "+v"(acc)                                                                 \
                    : "v"(x), "v"(y));                                                          \
        else                                                                                    \
            __asm__("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #L                                \
                    " row_mask:0xf bank_mask:0xf"                                               \
                    : "+v"(acc)                                                                 \
                    : "v"(x), "v"(y));                                                          \
        break;
        SS_FMAC_BCAST(0) SS_FMAC_BCAST(1) SS_FMAC_BCAST(2) SS_FMAC_BCAST(3)
        SS_FMAC_BCAST(4) SS_FMAC_BCAST(5) SS_FMAC_BCAST(6) SS_FMAC_BCAST(7)
        SS_FMAC_BCAST(8) SS_FMAC_BCAST(9) SS_FMAC_BCAST(10) SS_FMAC_BCAST(11)
        SS_FMAC_BCAST(12) SS_FMAC_BCAST(13) SS_FMAC_BCAST(14) SS_FMAC_BCAST(15)
#undef SS_FMAC_BCAST
    }
    return acc;
}

// DPP lane permutations within a 16-lane row (one VALU op each, or folded
// into the add that consumes them): lane n reads lane n ^ 15 (row_mirror),
// n ^ 7 (row_half_mirror), n ^ 2 and n ^ 1 (quad_perm).
template <int CTRL>
__device__ __forceinline__ float dpp_lane(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// One butterfly level: `x` holds 2K values; the lane keeps one half (the low
// one when `low`) and adds the partner's copy of that half, which the partner
// sends in place of its own kept half.  Own value first.
template <int CTRL, int K>
__device__ __forceinline__ void fold_level(const float *x, float *out, bool low) {
#pragma unroll
    for (int i = 0; i < K; i++) {
        const float keep = low ? x[i] : x[K + i];
        const float send = low ? x[K + i] : x[i];
        out[i] = keep + dpp_lane<CTRL>(send);
    }
}

// The first two butterfly levels select by lane bit 3 and bit 2, which are
// the bits of the 4-lane bank within the row.  A DPP op does not write the
// lanes of the banks its bank_mask leaves out, so each fold is two DPP adds
// (one per kept half) and needs no select.  The sums are the same as
// fold_level's (own + partner and partner + own are the same float).  One
// s_nop 1 in front of each block gives the two wait states a DPP read needs
// after the VALU op that wrote its source; within a block no DPP op reads a
// register the block wrote fewer than two instructions earlier.  (The
// compiler writes EXEC only with scalar instructions on this target, so the
// longer wait after a VALU write of EXEC does not arise.)
#define SS_FOLD2(CTRL, O, A, B, MA, MB)                                  \
    "v_add_f32_dpp %[" #O "], %[" #A "], %[" #A "] " CTRL " row_mask:0xf bank_mask:" MA "\n\t" \
    "v_add_f32_dpp %[" #O "], %[" #B "], %[" #B "] " CTRL " row_mask:0xf bank_mask:" MB "\n\t"

// level n ^ 15: banks 0, 1 keep lo, banks 2, 3 keep hi
__device__ __forceinline__ void fold_banks_mirror(const float (&lo)[8], const float (&hi)[8],
                                                  float (&out)[8]) {
    __asm__("s_nop 1\n\t"
            SS_FOLD2("row_mirror", o0, l0, h0, "0x3", "0xc")
            SS_FOLD2("row_mirror", o1, l1, h1, "0x3", "0xc")
            SS_FOLD2("row_mirror", o2, l2, h2, "0x3", "0xc")
            SS_FOLD2("row_mirror", o3, l3, h3, "0x3", "0xc")
            SS_FOLD2("row_mirror", o4, l4, h4, "0x3", "0xc")
            SS_FOLD2("row_mirror", o5, l5, h5, "0x3", "0xc")
            SS_FOLD2("row_mirror", o6, l6, h6, "0x3", "0xc")
            SS_FOLD2("row_mirror", o7, l7, h7, "0x3", "0xc")
            : [o0] "=&v"(out[0]), [o1] "=&v"(out[1]), [o2] "=&v"(out[2]), [o3] "=&v"(out[3]),
              [o4] "=&v"(out[4]), [o5] "=&v"(out[5]), [o6] "=&v"(out[6]), [o7] "=&v"(out[7])
            : [l0] "v"(lo[0]), [l1] "v"(lo[1]), [l2] "v"(lo[2]), [l3] "v"(lo[3]),
              [l4] "v"(lo[4]), [l5] "v"(lo[5]), [l6] "v"(lo[6]), [l7] "v"(lo[7]),
              [h0] "v"(hi[0]), [h1] "v"(hi[1]), [h2] "v"(hi[2]), [h3] "v"(hi[3]),
              [h4] "v"(hi[4]), [h5] "v"(hi[5]), [h6] "v"(hi[6]), [h7] "v"(hi[7]));
}

// level n ^ 7: banks 0, 2 keep x[0..3], banks 1, 3 keep x[4..7]
__device__ __forceinline__ void fold_banks_half_mirror(const float (&x)[8], float (&out)[4]) {
    __asm__("s_nop 1\n\t"
            SS_FOLD2("row_half_mirror", o0, a0, b0, "0x5", "0xa")
            SS_FOLD2("row_half_mirror", o1, a1, b1, "0x5", "0xa")
            SS_FOLD2("row_half_mirror", o2, a2, b2, "0x5", "0xa")
            SS_FOLD2("row_half_mirror", o3, a3, b3, "0x5", "0xa")
            : [o0] "=&v"(out[0]), [o1] "=&v"(out[1]), [o2] "=&v"(out[2]), [o3] "=&v"(out[3])
            : [a0] "v"(x[0]), [a1] "v"(x[1]), [a2] "v"(x[2]), [a3] "v"(x[3]),
              [b0] "v"(x[4]), [b1] "v"(x[5]), [b2] "v"(x[6]), [b3] "v"(x[7]));
}
#undef SS_FOLD2

// The same sum as row_transpose_sum, for a lane that already holds the 16
// terms (x[k] = term of lane k): the butterfly's grouping depends only on the
// lane masks, so it is one fixed tree over k -- pairs {k, 15 - k}, joined
// with {k ^ 7, k ^ 8}, then across k ^ 2, then k ^ 1 -- and this returns the
// same bits.
__device__ __forceinline__ float row_tree_sum(const float (&x)[16]) {
    float a[8], b[4];
#pragma unroll
    for (int k = 0; k < 8; k++) a[k] = x[k] + x[15 - k];
#pragma unroll
    for (int k = 0; k < 4; k++) b[k] = a[k] + a[7 - k];
    return (b[0] + b[2]) + (b[1] + b[3]);
}

// Sum over the 16 lanes of a DPP row of 16 values per lane, all in
// registers: lane n ends with the sum of value n (lo[n] for n < 8, hi[n - 8]
// otherwise).  Four butterfly levels pair lanes n ^ 15, n ^ 7, n ^ 2 and
// n ^ 1; those masks generate all 16 lanes and each level joins disjoint
// lane sets, so every lane's value is added exactly once, in an order fixed
// by the lane index.
__device__ __forceinline__ float row_transpose_sum(const float (&lo)[8], const float (&hi)[8],
                                                   int n) {
    float x8[8], x4[4], x2[2], x1[1];
    fold_banks_mirror(lo, hi, x8);                  // row_mirror: n ^ 15
    fold_banks_half_mirror(x8, x4);                 // row_half_mirror: n ^ 7
    fold_level<0x4E, 2>(x4, x2, (n & 3) < 2);      // quad_perm [2,3,0,1]: n ^ 2
    fold_level<0xB1, 1>(x2, x1, (n & 1) == 0);     // quad_perm [1,0,3,2]: n ^ 1
    return x1[0];
}

template <int M>
__device__ __forceinline__ float xor_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                     (M << 10) | 0x1f));
}

// Sum over the 16 lanes of a DPP row; pairs are combined commutatively, so
// every lane of the row ends with the same bits.
__device__ __forceinline__ float row_sum16(float v) {
    return xor_add<8>(xor_add<4>(xor_add<2>(xor_add<1>(v))));
}

}  // namespace ssk
