// ss_conv_lane.h -- the causal convolution fused into the scan kernels.
//
// The Mamba block of the state-spaces/mamba README ("Usage", Mamba block)
// runs a width-d_conv (4) causal convolution over each channel right in
// front of the selective scan.  Fused, the scan's u is never stored: the
// lane that owns element t of its row (step n of a 16-step block) forms
//   pre_t = bias + sum_k w[k] x_{t-H+k},   H = K - 1,   u_t = act(pre_t),
// the taps added in ascending k as the convolution kernel adds them, and
// rounds u to the io type as that kernel stores it, so a fused call and
// the convolution kernel followed by the scan give the same bits (and the
// backward recomputes the forward's u exactly).  The inputs at lags 1..3
// come from lanes n - 1 .. n - 3 of the same DPP row, or of the previous
// block for the first lanes; the backward's input gradient needs the
// pre-activation gradients at leads 1..3, from lanes n + 1 .. n + 3 or the
// next block.
#pragma once

#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_tiles.h"

namespace ssk {

struct ConvLane {
    float wl[kConvMaxWidth];   // weight of lag j (tap K - 1 - j); zero past K
    float b;
    int K;
    bool silu;
};

// P: FwdParams or BwdParams (conv_width, conv_silu, conv_w, conv_b)
template <typename P>
__device__ __forceinline__ ConvLane conv_lane(const P &p, int64_t d, bool row_ok) {
    ConvLane c;
    c.K = p.conv_width;
    c.silu = p.conv_silu != 0;
    c.b = (row_ok && p.conv_b) ? p.conv_b[d] : 0.0f;
#pragma unroll
    for (int j = 0; j < kConvMaxWidth; j++)
        c.wl[j] = (row_ok && j < c.K) ? p.conv_w[d * c.K + (c.K - 1 - j)] : 0.0f;
    return c;
}

// lane n of a DPP row: `cur` of lane n - J when n >= J, else `prev` of lane
// n + 16 - J (a rotate of prev, then a shift of cur whose out-of-row source
// lanes keep the rotated value)
template <int J>
__device__ __forceinline__ float lagged(float cur, float prev) {
    // a rotate never leaves the row, so it needs no old value
    const int o = __builtin_amdgcn_mov_dpp(__float_as_int(prev), 0x120 + J, 0xf, 0xf, false);
    return __int_as_float(
        __builtin_amdgcn_update_dpp(o, __float_as_int(cur), 0x110 + J, 0xf, 0xf, false));
}

// lane n of a DPP row: `cur` of lane n + J when n + J < 16, else `next` of
// lane n + J - 16 (a rotate of next by 16 - J, then a left shift of cur)
template <int J>
__device__ __forceinline__ float led(float cur, float next) {
    const int o = __builtin_amdgcn_mov_dpp(__float_as_int(next), 0x120 + 16 - J, 0xf, 0xf, false);
    return __int_as_float(
        __builtin_amdgcn_update_dpp(o, __float_as_int(cur), 0x100 + J, 0xf, 0xf, false));
}

// The pre-activation of the lane's element (x its input, prev the lane's
// input one block -- 16 steps -- earlier) and its inputs by lag, xl[j] =
// x_{t-j}.  KC: the width when fixed at compile time (4, the Mamba
// block's), else 0 and c.K is read at run time.
template <int KC>
__device__ __forceinline__ float conv_pre(const ConvLane &c, float x, float prev,
                                          float (&xl)[kConvMaxWidth]) {
    const int K = KC > 0 ? KC : c.K;
    xl[0] = x;
    xl[1] = K >= 2 ? lagged<1>(x, prev) : 0.0f;
    xl[2] = K >= 3 ? lagged<2>(x, prev) : 0.0f;
    xl[3] = K == 4 ? lagged<3>(x, prev) : 0.0f;
    float acc = c.b;
    if (K == 4) acc = __builtin_fmaf(c.wl[3], xl[3], acc);
    if (K >= 3) acc = __builtin_fmaf(c.wl[2], xl[2], acc);
    if (K >= 2) acc = __builtin_fmaf(c.wl[1], xl[1], acc);
    return __builtin_fmaf(c.wl[0], x, acc);
}

// u from the pre-activation, rounded to the io type
template <typename T>
__device__ __forceinline__ float conv_act(const ConvLane &c, float pre) {
    const float u = c.silu ? pre * sigmoid_f32(pre) : pre;
    return to_f32<T>(from_f32<T>(u));
}

// d act / d pre
__device__ __forceinline__ float conv_act_grad(const ConvLane &c, float pre) {
    if (!c.silu) return 1.0f;
    const float s = sigmoid_f32(pre);
    return s * (1.0f + pre * (1.0f - s));
}

template <typename T, int KC>
__device__ __forceinline__ float conv_u(const ConvLane &c, float x, float prev) {
    float xl[kConvMaxWidth];
    return conv_act<T>(c, conv_pre<KC>(c, x, prev, xl));
}

// The input gradient of the lane's element from the pre-activation
// gradients g (this block) and gnext (the next block, 16 steps later):
// dx_t = sum_j wl[j] g_{t+j}, j ascending.
template <int KC>
__device__ __forceinline__ float conv_dx(const ConvLane &c, float g, float gnext) {
    const int K = KC > 0 ? KC : c.K;
    float acc = c.wl[0] * g;
    if (K >= 2) acc = __builtin_fmaf(c.wl[1], led<1>(g, gnext), acc);
    if (K >= 3) acc = __builtin_fmaf(c.wl[2], led<2>(g, gnext), acc);
    if (K == 4) acc = __builtin_fmaf(c.wl[3], led<3>(g, gnext), acc);
    return acc;
}

// The input the lane would hold one block before step t0: x of row (b, d)
// at t0 - 16 + n, the initial window for the H steps before 0, else zero.
// P: FwdParams or BwdParams (u holds x).
template <typename T, typename P>
__device__ __forceinline__ float conv_prev(const P &p, int64_t b, int64_t d, bool row_ok,
                                           int64_t t0, int n) {
    const int64_t t = t0 - 16 + n;
    const int H = p.conv_width - 1;
    if (!row_ok || t < -H) return 0.0f;
    if (t >= 0) return to_f32<T>(ld_global(static_cast<const T *>(p.u) + (b * p.dim + d) * p.seqlen + t));
    return p.conv_init ? p.conv_init[(b * p.dim + d) * H + (t + H)] : 0.0f;
}

// The same input as conv_prev, in two parts that need no arithmetic on a
// load result where the load is issued (a loop can issue it a chunk ahead
// and take it a chunk later without draining the loads behind it):
// conv_prev_bits loads the raw io-type bits of x at max(t0 - 16 + n, 0) of
// the row (row 0 of the batch entry past the last channel), unconditionally;
// conv_window gives the initial-window value for t0 = 0.
template <typename T>
using ConvBits = std::conditional_t<sizeof(T) == 4, uint32_t, uint16_t>;

template <typename T, typename P>
__device__ __forceinline__ ConvBits<T> conv_prev_bits(const P &p, int64_t b, int64_t d, bool row_ok,
                                                      int64_t t0, int n) {
    const int64_t t = t0 - 16 + n;
    const ConvBits<T> *xr =
        static_cast<const ConvBits<T> *>(p.u) + (b * p.dim + (row_ok ? d : 0)) * p.seqlen;
    return ld_global(xr + (t > 0 ? t : 0));
}
// (kept in the io type's width, a 2-byte value needs no zero extension
// before the shift that widens it)
template <typename T>
__device__ __forceinline__ float conv_bits_f32(ConvBits<T> bitsv) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(bitsv);
    else return __uint_as_float(uint32_t(bitsv) << 16);
}
template <typename P>
__device__ __forceinline__ float conv_window(const P &p, int64_t b, int64_t d, bool row_ok, int n) {
    const int H = p.conv_width - 1;
    return (row_ok && p.conv_init && n >= 16 - H) ? p.conv_init[(b * p.dim + d) * H + (n - (16 - H))]
                                                  : 0.0f;
}

}  // namespace ssk
