// ss_state_update.hip -- one-token state update (decode step) for gfx950.
//
// Advances the carried state of every (batch b, channel d) row by one step
// of the recurrence and emits that step's output (the single-token step on
// a carried state of the mamba-rs README, "Quick start (CPU)"):
//   h[n] <- exp(delta A[d,n]) h[n] + delta B[b,n] u ;  y = (sum_n C[b,n] h[n] + D u) silu(z)
//
// The step is bound by HBM traffic on the f32 state (64 bytes read and 64
// written per row and 16 states).  Four lanes own one row, each a float4 of
// every 16-state slice, so a wavefront streams 16 rows x 64 bytes of
// contiguous state per access.  The
// output sum runs in a fixed order (4 states in-lane, then a 2-level
// butterfly whose partial sums are combined commutatively), so every lane of
// a row -- and every batch size -- produces the same bits.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ssk {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 4;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;

template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (MASK << 10) | 0x1f));
}

// State entries 16 k + 4 q .. 16 k + 4 q + 3 of every 16-state slice k
// belong to lane q of the row.  kFull: dstate a multiple of 16, so every
// lane moves a float4 per slice.  Otherwise the same lanes and sums with
// element loads, states n >= dstate held at zero.
template <typename T, bool kFull>
__global__ __launch_bounds__(kThreads) void ss_state_update_kernel(DecodeParams p) {
    const int64_t rows = p.batch * p.dim;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 2);
    const int q = threadIdx.x & 3;  // which float4 of each 16-entry slice
    const bool ok = row < rows;
    const int64_t rr = ok ? row : 0;
    const int64_t b = rr / p.dim;
    const int64_t d = rr - b * p.dim;
    const int Ns = p.nstate;
    const int slices = state_slices(Ns);

    const T *gu = static_cast<const T *>(p.u);
    const T *gdl = static_cast<const T *>(p.delta);
    const T *gz = static_cast<const T *>(p.z);
    const T *gB = static_cast<const T *>(p.B);
    const T *gC = static_cast<const T *>(p.C);

    float uu = 0.f, dlr = 0.f, zz = 0.f, bias = 0.f, dskip = 0.f;
    if (ok) {
        uu = to_f32<T>(gu[rr]);
        dlr = to_f32<T>(gdl[rr]);
        if (p.z) zz = to_f32<T>(gz[rr]);
        if (p.bias) bias = p.bias[d];
        if (p.D) dskip = p.D[d];
    }
    float dl = dlr + bias;
    if (p.softplus) dl = softplus_f32(dl);
    const float dlu = dl * uu;
    float part = 0.0f;
    for (int k = 0; k < slices; k++) {
        const int n0 = 16 * k + 4 * q;
        float hv[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
        float bb[4] = {0.f, 0.f, 0.f, 0.f}, cc[4] = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
            if constexpr (kFull) {
                const float4 h4 = reinterpret_cast<const float4 *>(p.state + rr * Ns)[n0 / 4];
                const float4 a4 = reinterpret_cast<const float4 *>(p.A + d * Ns)[n0 / 4];
                hv[0] = h4.x; hv[1] = h4.y; hv[2] = h4.z; hv[3] = h4.w;
                av[0] = a4.x; av[1] = a4.y; av[2] = a4.z; av[3] = a4.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (n0 + e < Ns) {
                        hv[e] = p.state[rr * Ns + n0 + e];
                        av[e] = p.A[d * Ns + n0 + e];
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if (kFull || n0 + e < Ns) {
                    bb[e] = to_f32<T>(gB[b * Ns + n0 + e]);
                    cc[e] = to_f32<T>(gC[b * Ns + n0 + e]);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            hv[e] = __builtin_fmaf(exp2_hw(dl * (av[e] * kLog2e)), hv[e], dlu * bb[e]);
            part = __builtin_fmaf(cc[e], hv[e], part);
        }
        if (ok) {
            if constexpr (kFull) {
                reinterpret_cast<float4 *>(p.state + rr * Ns)[n0 / 4] =
                    make_float4(hv[0], hv[1], hv[2], hv[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    if (n0 + e < Ns) p.state[rr * Ns + n0 + e] = hv[e];
            }
        }
    }
    // lanes 4k..4k+3 hold one row: ((p0 + p1) + (p2 + p3)) on every lane
    part += xor_lane<1>(part);
    part += xor_lane<2>(part);
    if (ok && q == 0) {
        float y = part + dskip * uu;
        if (p.z) y *= zz * sigmoid_f32(zz);
        static_cast<T *>(p.out)[rr] = from_f32<T>(y);
    }
}

}  // namespace

hipError_t launch_state_update(const DecodeParams &p, bool bf16, hipStream_t stream) {
    const int64_t rows = p.batch * p.dim;
    if (rows == 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    const bool full = p.nstate % kN == 0;
    if (bf16 && full)
        hipLaunchKernelGGL((ss_state_update_kernel<bf16_t, true>), grid, dim3(kThreads), 0, stream, p);
    else if (bf16)
        hipLaunchKernelGGL((ss_state_update_kernel<bf16_t, false>), grid, dim3(kThreads), 0, stream, p);
    else if (full)
        hipLaunchKernelGGL((ss_state_update_kernel<float, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((ss_state_update_kernel<float, false>), grid, dim3(kThreads), 0, stream, p);
    profile_mark(stream);
    return hipGetLastError();
}

}  // namespace ssk
