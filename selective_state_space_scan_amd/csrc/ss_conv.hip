// ss_conv.hip -- causal depthwise convolution over time (+ SiLU) for gfx950.
//
// The Mamba block of the state-spaces/mamba README ("Usage", Mamba block)
// runs a local convolution of width d_conv = 4 along time over each channel
// before the selective scan, and the mamba-rs README ("Quick start (CPU)")
// keeps its window in the decode state.  For row (b, d), with K = width and
// H = K - 1:
//   pre_t = bias[d] + sum_{k<K} w[d,k] x_{t-H+k},   out_t = silu(pre_t) or pre_t
// where x_{-H..-1} come from the initial window (zeros without one).
//
// Work layout.  A row is cut into segments of kConvSeg steps, one wavefront
// per segment.  On the vector path (seqlen a multiple of the 16-byte vector
// of V elements) lane l holds, at step j of its segment, the vector of
// elements t0 + (64 j + l) V .. + V - 1; every load and store is one
// coalesced 16-byte access per lane.  The H inputs in front of a vector are
// the tail of lane l-1's vector: one wave-rotate DPP move per word (lane 0
// takes lane 63's vector of the previous step, and the segment's first
// vector a halo read from memory or from the initial window).  The
// backward's input gradient needs the H output gradients behind a vector,
// which come from lane l+1 the same way.  Lengths that are not a multiple
// of V take a per-element path that reads each window from memory.
//
// The HBM traffic is the algorithmic one: the forward reads x and writes
// out once; the backward reads x and dout and writes dx once, and sums the
// weight and bias gradients on chip (one workgroup per channel).
#include <type_traits>

#include "ss_kernels.h"
#include "ss_device.h"
#include "ss_tiles.h"

namespace ssk {

namespace {

constexpr int kConvSeg = 2048;  // steps per segment (one wavefront)
constexpr int kConvWaves = 4;   // wavefronts per workgroup

template <typename T>
struct VecOf {
    static constexpr int n = 16 / int(sizeof(T));
};

// Element i of a 16-byte vector of T, widened to f32 (i is a constant once
// the surrounding loops are unrolled).
template <typename T>
__device__ __forceinline__ float vget(const u32x4 &v, int i) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(v[i]);
    } else {
        const uint32_t w = v[i >> 1];
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
}

template <typename T, int V>
__device__ __forceinline__ u32x4 vpack(const float (&o)[V]) {
    u32x4 r;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < 4; i++) r[i] = __float_as_uint(o[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
            r[i] = uint32_t(f32_to_bf16(o[2 * i])) | (uint32_t(f32_to_bf16(o[2 * i + 1])) << 16);
    }
    return r;
}

// Lane l receives lane l-1's value (lane 0 receives lane 63's).
__device__ __forceinline__ uint32_t wave_ror1(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x13C, 0xf, 0xf, false));
}
// Lane l receives lane l+1's value (lane 63 receives lane 0's).
__device__ __forceinline__ float wave_rol1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x134, 0xf, 0xf, false));
}

template <bool SILU>
__device__ __forceinline__ float act(float pre) {
    return SILU ? pre * sigmoid_f32(pre) : pre;
}
// d act / d pre:  silu'(p) = s (1 + p (1 - s)),  s = sigmoid(p)
template <bool SILU>
__device__ __forceinline__ float act_grad(float pre) {
    if constexpr (SILU) {
        const float s = sigmoid_f32(pre);
        return s * (1.0f + pre * (1.0f - s));
    } else {
        return 1.0f;
    }
}

// What a wavefront works on: row r = b * dim + d, segment seg of that row.
struct ConvWave {
    int64_t r, d, seg, t0;
    bool live;
};

__device__ __forceinline__ ConvWave conv_wave(const ConvParams &p, int64_t nseg) {
    ConvWave w;
    const int64_t wave = int64_t(blockIdx.x) * kConvWaves + (threadIdx.x >> 6);
    const int64_t rows = p.batch * p.dim;
    w.live = wave < rows * nseg;
    w.r = wave / nseg;
    w.seg = wave - w.r * nseg;
    w.d = w.r % p.dim;
    w.t0 = w.seg * kConvSeg;
    return w;
}

// Input at step tt of row r (tt >= -H): x, or the initial window, or zero.
template <typename T, int H>
__device__ __forceinline__ float x_at(const ConvParams &p, const T *xr, int64_t r, int64_t tt) {
    if (tt >= 0) return to_f32(ld_global(xr + tt));
    return p.init ? ld_global(p.init + r * H + (tt + H)) : 0.0f;
}

// Final window of row r: the inputs at steps L-H .. L-1 (lanes 0..H-1).
template <typename T, int H>
__device__ __forceinline__ void write_final(const ConvFwdParams &p, const T *xr, int64_t r,
                                            int lane) {
    if (H > 0 && lane < H) p.final_state[r * H + lane] = x_at<T, H>(p, xr, r, p.seqlen - H + lane);
}

// Sum over the 64 lanes in a fixed butterfly order; lane 0's result is used.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, int K, bool SILU>
__global__ __launch_bounds__(64 * kConvWaves) void conv_fwd_vec(ConvFwdParams p, int64_t nseg) {
    constexpr int V = VecOf<T>::n, H = K - 1, J = kConvSeg / (64 * V);
    constexpr int HS = H > 0 ? H : 1;
    constexpr int W0 = ((V - HS) * int(sizeof(T))) / 4;  // first word holding the tail
    const int lane = threadIdx.x & 63;
    const ConvWave cw = conv_wave(p, nseg);
    if (!cw.live) return;
    const int64_t L = p.seqlen;
    const T *xr = static_cast<const T *>(p.x) + cw.r * L;
    T *orow = static_cast<T *>(p.out) + cw.r * L;
    if (p.final_state && cw.seg == nseg - 1) write_final<T, H>(p, xr, cw.r, lane);
    if (cw.t0 >= L) return;

    float w[K];
#pragma unroll
    for (int k = 0; k < K; k++) w[k] = p.w[cw.d * K + k];
    const float b = p.bias ? p.bias[cw.d] : 0.0f;

    // Vectors past the row end load the row's last vector and are not stored.
    u32x4 v[J];
#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t t = cw.t0 + int64_t(j * 64 + lane) * V;
        v[j] = ld_global16(at_bytes(xr, uint32_t((t < L ? t : L - V) * int64_t(sizeof(T)))));
    }
    float carry[HS];
#pragma unroll
    for (int m = 0; m < H; m++) carry[m] = x_at<T, H>(p, xr, cw.r, cw.t0 - H + m);

#pragma unroll
    for (int j = 0; j < J; j++) {
        const int64_t t = cw.t0 + int64_t(j * 64 + lane) * V;
        u32x4 rv = v[j];
#pragma unroll
        for (int q = W0; q < 4; q++) rv[q] = wave_ror1(v[j][q]);
        float prev[HS];
#pragma unroll
        for (int m = 0; m < H; m++) {
            const float rot = vget<T>(rv, V - H + m);
            prev[m] = lane == 0 ? carry[m] : rot;
            carry[m] = rot;
        }
        float o[V];
#pragma unroll
        for (int e = 0; e < V; e++) {
            float acc = b;
#pragma unroll
            for (int k = 0; k < K; k++) {
                const int i = e - H + k;
                acc = fmaf(w[k], i >= 0 ? vget<T>(v[j], i) : prev[H + i], acc);
            }
            o[e] = act<SILU>(acc);
        }
        if (t < L) st_global16(at_bytes(orow, uint32_t(t * int64_t(sizeof(T)))), vpack<T, V>(o));
    }
}

template <typename T, int K, bool SILU>
__global__ __launch_bounds__(64 * kConvWaves) void conv_fwd_elem(ConvFwdParams p, int64_t nseg) {
    constexpr int H = K - 1;
    const int lane = threadIdx.x & 63;
    const ConvWave cw = conv_wave(p, nseg);
    if (!cw.live) return;
    const int64_t L = p.seqlen;
    const T *xr = static_cast<const T *>(p.x) + cw.r * L;
    T *orow = static_cast<T *>(p.out) + cw.r * L;
    if (p.final_state && cw.seg == nseg - 1) write_final<T, H>(p, xr, cw.r, lane);
    float w[K];
#pragma unroll
    for (int k = 0; k < K; k++) w[k] = p.w[cw.d * K + k];
    const float b = p.bias ? p.bias[cw.d] : 0.0f;
    for (int j = 0; j < kConvSeg / 64; j++) {
        const int64_t t = cw.t0 + j * 64 + lane;
        if (cw.t0 + j * 64 >= L) break;
        if (t < L) {
            float acc = b;
#pragma unroll
            for (int k = 0; k < K; k++) acc = fmaf(w[k], x_at<T, H>(p, xr, cw.r, t - H + k), acc);
            st_global(orow + t, from_f32<T>(act<SILU>(acc)));
        }
    }
}

// ---------------------------------------------------------------------------
// backward: g_t = dout_t act'(pre_t);  dx_s = sum_k w[k] g_{s+H-k};
// dw[k] = sum g_t x_{t-H+k};  dbias = sum g_t;  dinit_j = sum_{k<=j} w[k] g_{j-k}
//
// One workgroup per channel d.  Its wavefronts take the (batch, segment)
// items of the channel in turn (wavefront v: items v, v + W, ...), keep the
// dw / dbias sums in registers across items, and the workgroup adds the
// per-wavefront sums in ascending order at the end: no partial buffer and
// no second kernel.  The order depends on the shape only.
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 2;  // wavefronts per workgroup (one channel)

// One (row, segment) item on the vector path: writes dx (and dinit for the
// first segment) and adds the item's dw / dbias sums to acc_w / acc_b.
template <typename T, int K, bool SILU>
__device__ __forceinline__ void bwd_vec_item(const ConvBwdParams &p, const float (&w)[K], float b,
                                             int64_t r, int64_t seg, int lane, float (&acc_w)[K],
                                             float &acc_b) {
    constexpr int V = VecOf<T>::n, H = K - 1, J = kConvSeg / (64 * V);
    constexpr int HS = H > 0 ? H : 1;
    constexpr int W0 = ((V - HS) * int(sizeof(T))) / 4;
    const int64_t L = p.seqlen;
    const int64_t t0 = seg * kConvSeg;
    const T *xr = static_cast<const T *>(p.x) + r * L;
    const T *gr = static_cast<const T *>(p.dout) + r * L;
    T *dxr = static_cast<T *>(p.dx) + r * L;

    if (t0 < L) {
        u32x4 v[J], go[J];
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int64_t t = t0 + int64_t(j * 64 + lane) * V;
            const uint32_t off = uint32_t((t < L ? t : L - V) * int64_t(sizeof(T)));
            v[j] = ld_global16(at_bytes(xr, off));
            go[j] = ld_global16(at_bytes(gr, off));
        }
        float carry[HS];
#pragma unroll
        for (int m = 0; m < H; m++) carry[m] = x_at<T, H>(p, xr, r, t0 - H + m);

        // gradients at the pre-activation, zero past the row end
        float g[J][V];
#pragma unroll
        for (int j = 0; j < J; j++) {
            const int64_t t = t0 + int64_t(j * 64 + lane) * V;
            u32x4 rv = v[j];
#pragma unroll
            for (int q = W0; q < 4; q++) rv[q] = wave_ror1(v[j][q]);
            float prev[HS];
#pragma unroll
            for (int m = 0; m < H; m++) {
                const float rot = vget<T>(rv, V - H + m);
                prev[m] = lane == 0 ? carry[m] : rot;
                carry[m] = rot;
            }
#pragma unroll
            for (int e = 0; e < V; e++) {
                float xw[K];
                float pre = b;
#pragma unroll
                for (int k = 0; k < K; k++) {
                    const int i = e - H + k;
                    xw[k] = i >= 0 ? vget<T>(v[j], i) : prev[H + i];
                    pre = fmaf(w[k], xw[k], pre);
                }
                const float gg = t < L ? vget<T>(go[j], e) * act_grad<SILU>(pre) : 0.0f;
                g[j][e] = gg;
                acc_b += gg;
#pragma unroll
                for (int k = 0; k < K; k++) acc_w[k] = fmaf(gg, xw[k], acc_w[k]);
            }
        }

        // the next segment's first H gradients (lane 63 of the last step reads them)
        float gnext[HS];
#pragma unroll
        for (int m = 0; m < H; m++) {
            const int64_t tt = t0 + kConvSeg + m;
            float gg = 0.0f;
            if (tt < L) {
                float pre = b;
#pragma unroll
                for (int k = 0; k < K; k++)
                    pre = fmaf(w[k], to_f32(ld_global(xr + (tt - H + k))), pre);
                gg = to_f32(ld_global(gr + tt)) * act_grad<SILU>(pre);
            }
            gnext[m] = gg;
        }

        // the first H gradients of lane l+1's vector, for every step
        float nr[J][HS];
#pragma unroll
        for (int j = 0; j < J; j++)
#pragma unroll
            for (int m = 0; m < H; m++) nr[j][m] = wave_rol1(g[j][m]);

#pragma unroll
        for (int j = 0; j < J; j++) {
            const int64_t t = t0 + int64_t(j * 64 + lane) * V;
            float nxt[HS];
#pragma unroll
            for (int m = 0; m < H; m++)
                nxt[m] = lane == 63 ? (j + 1 < J ? nr[j + 1][m] : gnext[m]) : nr[j][m];
            float o[V];
#pragma unroll
            for (int e = 0; e < V; e++) {
                float acc = 0.0f;
#pragma unroll
                for (int k = K - 1; k >= 0; k--) {
                    const int i = e + H - k;
                    acc = fmaf(w[k], i < V ? g[j][i] : nxt[i - V], acc);
                }
                o[e] = acc;
            }
            if (t < L) st_global16(at_bytes(dxr, uint32_t(t * int64_t(sizeof(T)))), vpack<T, V>(o));
        }

        if (p.dinit && seg == 0 && lane == 0) {
#pragma unroll
            for (int jj = 0; jj < H; jj++) {
                float acc = 0.0f;
#pragma unroll
                for (int k = jj; k >= 0; k--) acc = fmaf(w[k], g[0][jj - k], acc);
                p.dinit[r * H + jj] = acc;
            }
        }
    } else if (p.dinit && H > 0 && lane < H) {
        p.dinit[r * H + lane] = 0.0f;  // empty rows: no gradient reaches the window
    }
}

template <typename T, int K, bool SILU>
__device__ __forceinline__ float g_at(const ConvBwdParams &p, const T *xr, const T *gr,
                                      const float (&w)[K], float b, int64_t r, int64_t tt) {
    constexpr int H = K - 1;
    if (tt >= p.seqlen) return 0.0f;
    float pre = b;
#pragma unroll
    for (int k = 0; k < K; k++) pre = fmaf(w[k], x_at<T, H>(p, xr, r, tt - H + k), pre);
    return to_f32(ld_global(gr + tt)) * act_grad<SILU>(pre);
}

template <typename T, int K, bool SILU>
__device__ __forceinline__ void bwd_elem_item(const ConvBwdParams &p, const float (&w)[K], float b,
                                              int64_t r, int64_t seg, int lane,
                                              float (&acc_w)[K], float &acc_b) {
    constexpr int H = K - 1;
    const int64_t L = p.seqlen;
    const int64_t t0 = seg * kConvSeg;
    const T *xr = static_cast<const T *>(p.x) + r * L;
    const T *gr = static_cast<const T *>(p.dout) + r * L;
    T *dxr = static_cast<T *>(p.dx) + r * L;
    for (int j = 0; j < kConvSeg / 64; j++) {
        const int64_t t = t0 + j * 64 + lane;
        if (t0 + j * 64 >= L) break;
        if (t < L) {
            const float gt = g_at<T, K, SILU>(p, xr, gr, w, b, r, t);
            acc_b += gt;
#pragma unroll
            for (int k = 0; k < K; k++)
                acc_w[k] = fmaf(gt, x_at<T, H>(p, xr, r, t - H + k), acc_w[k]);
            float acc = 0.0f;
#pragma unroll
            for (int k = K - 1; k >= 0; k--)
                acc = fmaf(w[k], k == H ? gt : g_at<T, K, SILU>(p, xr, gr, w, b, r, t + H - k),
                           acc);
            st_global(dxr + t, from_f32<T>(acc));
        }
    }
    if (p.dinit && seg == 0 && H > 0 && lane < H) {
        float acc = 0.0f;
#pragma unroll
        for (int k = K - 1; k >= 0; k--)
            if (k <= lane) acc = fmaf(w[k], g_at<T, K, SILU>(p, xr, gr, w, b, r, lane - k), acc);
        p.dinit[r * H + lane] = acc;
    }
}

// The backward kernel: workgroup = channel d, see above.
template <typename T, int K, bool SILU, bool VEC>
__global__ __launch_bounds__(64 * kBwdWaves) void conv_bwd_kernel(ConvBwdParams p, int64_t nseg) {
    __shared__ float red[kBwdWaves][K + 1];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t d = blockIdx.x;
    float w[K], acc_w[K], acc_b = 0.0f;
#pragma unroll
    for (int k = 0; k < K; k++) {
        w[k] = p.w[d * K + k];
        acc_w[k] = 0.0f;
    }
    const float b = p.bias ? p.bias[d] : 0.0f;
    const int64_t items = p.batch * nseg;
    for (int64_t it = wv; it < items; it += kBwdWaves) {
        const int64_t bb = it / nseg, seg = it - bb * nseg;
        if constexpr (VEC)
            bwd_vec_item<T, K, SILU>(p, w, b, bb * p.dim + d, seg, lane, acc_w, acc_b);
        else
            bwd_elem_item<T, K, SILU>(p, w, b, bb * p.dim + d, seg, lane, acc_w, acc_b);
    }
    float sum[K + 1];
#pragma unroll
    for (int k = 0; k < K; k++) sum[k] = wave_sum(acc_w[k]);
    sum[K] = wave_sum(acc_b);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k <= K; k++) red[wv][k] = sum[k];
    }
    __syncthreads();
    if (threadIdx.x <= K) {
        const int k = threadIdx.x;
        float t = 0.0f;
#pragma unroll
        for (int v = 0; v < kBwdWaves; v++) t += red[v][k];
        if (k < K) p.dw[d * K + k] = t;
        else if (p.dbias) p.dbias[d] = t;
    }
}

// ---------------------------------------------------------------------------
// decode: one input per row; the window (state) shifts by one
// ---------------------------------------------------------------------------
template <typename T, int K, bool SILU>
__global__ __launch_bounds__(256) void conv_update_kernel(ConvUpdateParams p) {
    constexpr int H = K - 1;
    const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (r >= p.batch * p.dim) return;
    const int64_t d = r % p.dim;
    float s[H > 0 ? H : 1];
#pragma unroll
    for (int m = 0; m < H; m++) s[m] = p.state[r * H + m];
    const float xv = to_f32(ld_global(static_cast<const T *>(p.x) + r));
    float acc = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < K; k++) acc = fmaf(p.w[d * K + k], k < H ? s[k] : xv, acc);
    st_global(static_cast<T *>(p.out) + r, from_f32<T>(act<SILU>(acc)));
#pragma unroll
    for (int m = 0; m < H; m++) p.state[r * H + m] = m + 1 < H ? s[m + 1] : xv;
}

// ---------------------------------------------------------------------------
// dispatch over (dtype, width, activation)
// ---------------------------------------------------------------------------
template <typename P, typename F>
hipError_t by_width(const P &p, F &&f) {
    switch (p.width) {
        case 1: f(std::integral_constant<int, 1>{}); break;
        case 2: f(std::integral_constant<int, 2>{}); break;
        case 3: f(std::integral_constant<int, 3>{}); break;
        case 4: f(std::integral_constant<int, 4>{}); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

dim3 wave_grid(int64_t waves) {
    return dim3(static_cast<unsigned>((waves + kConvWaves - 1) / kConvWaves));
}

template <typename T>
hipError_t conv_fwd_typed(const ConvFwdParams &p, hipStream_t stream) {
    const int64_t nseg = conv_segments(p.seqlen);
    const dim3 grid = wave_grid(p.batch * p.dim * nseg), block(64 * kConvWaves);
    const bool vec = p.seqlen % VecOf<T>::n == 0;
    return by_width(p, [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        if (vec && p.silu)
            hipLaunchKernelGGL((conv_fwd_vec<T, K, true>), grid, block, 0, stream, p, nseg);
        else if (vec)
            hipLaunchKernelGGL((conv_fwd_vec<T, K, false>), grid, block, 0, stream, p, nseg);
        else if (p.silu)
            hipLaunchKernelGGL((conv_fwd_elem<T, K, true>), grid, block, 0, stream, p, nseg);
        else
            hipLaunchKernelGGL((conv_fwd_elem<T, K, false>), grid, block, 0, stream, p, nseg);
    });
}

template <typename T>
hipError_t conv_bwd_typed(const ConvBwdParams &p, hipStream_t stream) {
    const int64_t nseg = conv_segments(p.seqlen);
    const dim3 grid(static_cast<unsigned>(p.dim)), block(64 * kBwdWaves);
    const bool vec = p.seqlen % VecOf<T>::n == 0;
    return by_width(p, [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        if (vec && p.silu)
            hipLaunchKernelGGL((conv_bwd_kernel<T, K, true, true>), grid, block, 0, stream, p, nseg);
        else if (vec)
            hipLaunchKernelGGL((conv_bwd_kernel<T, K, false, true>), grid, block, 0, stream, p, nseg);
        else if (p.silu)
            hipLaunchKernelGGL((conv_bwd_kernel<T, K, true, false>), grid, block, 0, stream, p, nseg);
        else
            hipLaunchKernelGGL((conv_bwd_kernel<T, K, false, false>), grid, block, 0, stream, p,
                               nseg);
    });
}

template <typename T>
hipError_t conv_update_typed(const ConvUpdateParams &p, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((p.batch * p.dim + 255) / 256)), block(256);
    return by_width(p, [&](auto kc) {
        constexpr int K = decltype(kc)::value;
        if (p.silu)
            hipLaunchKernelGGL((conv_update_kernel<T, K, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((conv_update_kernel<T, K, false>), grid, block, 0, stream, p);
    });
}

}  // namespace

int64_t conv_segments(int64_t seqlen) {
    return seqlen <= 0 ? 1 : (seqlen + kConvSeg - 1) / kConvSeg;
}

hipError_t launch_conv_fwd(const ConvFwdParams &p, bool bf16, hipStream_t stream) {
    if (p.batch * p.dim == 0) return hipSuccess;
    hipError_t e = bf16 ? conv_fwd_typed<bf16_t>(p, stream) : conv_fwd_typed<float>(p, stream);
    profile_mark(stream);
    return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_conv_bwd(const ConvBwdParams &p, bool bf16, hipStream_t stream) {
    if (p.dim == 0) return hipSuccess;
    hipError_t e = bf16 ? conv_bwd_typed<bf16_t>(p, stream) : conv_bwd_typed<float>(p, stream);
    profile_mark(stream);
    return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_conv_update(const ConvUpdateParams &p, bool bf16, hipStream_t stream) {
    if (p.batch * p.dim == 0) return hipSuccess;
    hipError_t e = bf16 ? conv_update_typed<bf16_t>(p, stream) : conv_update_typed<float>(p, stream);
    profile_mark(stream);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace ssk
