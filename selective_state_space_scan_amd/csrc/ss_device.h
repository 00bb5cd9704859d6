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
// within e^-20 relative.  Otherwise log1p(e) with e = e^x is evaluated as
// log(w) * e / (w - 1), w = 1 + e, which cancels the rounding of w and keeps
// the result accurate to a few ulp even when e is tiny (w == 1 gives e).
__device__ __forceinline__ float softplus_f32(float x) {
    float e = exp2_hw(x * kLog2e);
    float w = 1.0f + e;
    float wm1 = w - 1.0f;
    float lg = __builtin_amdgcn_logf(w) * kLn2;  // v_log_f32 is log2
    float r = (wm1 == 0.0f) ? e : lg * (e * __builtin_amdgcn_rcpf(wm1));
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

}  // namespace ssk
