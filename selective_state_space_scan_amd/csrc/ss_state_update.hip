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
// contiguous state per access; the state is read and written with
// non-temporal accesses (it is touched once), which measured 43 -> 37 us at
// 256 x 5120 against 30.5 us for a plain read-modify-write of the state
// alone.  The grid is (channel blocks, batch), so no lane divides.  The
// output sum runs in a fixed order (4 states in-lane, then a 2-level
// butterfly whose partial sums are combined commutatively), so every lane of
// a row -- and every batch size -- produces the same bits.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ssk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 4;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;

template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (MASK << 10) | 0x1f));
}

// Four consecutive B or C values of one batch entry, widened to f32.
template <typename T>
__device__ __forceinline__ void ld4_bc(const T *p, float (&v)[4]) {
    if constexpr (sizeof(T) == 4) {
        const float4 r = *reinterpret_cast<const float4 *>(p);
        v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    } else {
        const uint2 r = *reinterpret_cast<const uint2 *>(p);
        v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xffff0000u);
        v[2] = __uint_as_float(r.y << 16); v[3] = __uint_as_float(r.y & 0xffff0000u);
    }
}

// State entries 16 k + 4 q .. 16 k + 4 q + 3 of every 16-state slice k
// belong to lane q of the row.  Each 4-lane group takes kRpt rows, kRows
// apart (kRows = rows per kRpt-th of a block), and issues the loads of all
// of them before any arithmetic, so every lane keeps kRpt 16-byte state
// loads in flight.  kFull: dstate a multiple of 16, so every lane moves a
// float4 of state, A, and 4 consecutive B and C values per slice.
// Otherwise the same lanes and sums with element loads, states n >= dstate
// held at zero.
template <typename T, bool kFull, int kRpt>
__global__ __launch_bounds__(kThreads) void ss_state_update_kernel(DecodeParams p) {
    const int q = threadIdx.x & 3;  // which float4 of each 16-entry slice
    const int Ns = p.nstate;
    const int slices = state_slices(Ns);
    const T *gu = static_cast<const T *>(p.u);
    const T *gdl = static_cast<const T *>(p.delta);
    const T *gz = static_cast<const T *>(p.z);
    const T *gB = static_cast<const T *>(p.B);
    const T *gC = static_cast<const T *>(p.C);

    // grid: x = channel blocks of one batch entry, y = batch entry
    int64_t rr[kRpt], bb[kRpt], dd[kRpt];
    bool ok[kRpt];
    float uu[kRpt], dlr[kRpt], zz[kRpt], bias[kRpt], dskip[kRpt];
#pragma unroll
    for (int i = 0; i < kRpt; i++) {
        const int64_t d = (static_cast<int64_t>(blockIdx.x) * kRpt + i) * kRowsPerBlock +
                          (threadIdx.x >> 2);
        ok[i] = d < p.dim;
        bb[i] = blockIdx.y;
        dd[i] = ok[i] ? d : 0;
        rr[i] = bb[i] * p.dim + dd[i];
        uu[i] = dlr[i] = zz[i] = bias[i] = dskip[i] = 0.0f;
        if (ok[i]) {
            uu[i] = to_f32<T>(gu[rr[i]]);
            dlr[i] = to_f32<T>(gdl[rr[i]]);
            if (p.z) zz[i] = to_f32<T>(gz[rr[i]]);
            if (p.bias) bias[i] = p.bias[dd[i]];
            if (p.D) dskip[i] = p.D[dd[i]];
        }
    }
    float part[kRpt];
#pragma unroll
    for (int i = 0; i < kRpt; i++) part[i] = 0.0f;
    for (int k = 0; k < slices; k++) {
        const int n0 = 16 * k + 4 * q;
        float hv[kRpt][4], av[kRpt][4], bv[kRpt][4], cv[kRpt][4];
#pragma unroll
        for (int i = 0; i < kRpt; i++) {
#pragma unroll
            for (int e = 0; e < 4; e++) hv[i][e] = av[i][e] = bv[i][e] = cv[i][e] = 0.0f;
            if (!ok[i]) continue;
            if constexpr (kFull) {
                // the state streams through once: non-temporal accesses keep
                // it from displacing A, B and C in the caches
                const f32x4 hx = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4 *>(p.state + rr[i] * Ns) + n0 / 4);
                const float4 h4 = make_float4(hx.x, hx.y, hx.z, hx.w);
                const float4 a4 = reinterpret_cast<const float4 *>(p.A + dd[i] * Ns)[n0 / 4];
                hv[i][0] = h4.x; hv[i][1] = h4.y; hv[i][2] = h4.z; hv[i][3] = h4.w;
                av[i][0] = a4.x; av[i][1] = a4.y; av[i][2] = a4.z; av[i][3] = a4.w;
                ld4_bc<T>(gB + bb[i] * Ns + n0, bv[i]);
                ld4_bc<T>(gC + bb[i] * Ns + n0, cv[i]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (n0 + e < Ns) {
                        hv[i][e] = p.state[rr[i] * Ns + n0 + e];
                        av[i][e] = p.A[dd[i] * Ns + n0 + e];
                        bv[i][e] = to_f32<T>(gB[bb[i] * Ns + n0 + e]);
                        cv[i][e] = to_f32<T>(gC[bb[i] * Ns + n0 + e]);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kRpt; i++) {
            float dl = dlr[i] + bias[i];
            if (p.softplus) dl = softplus_f32(dl);
            const float dlu = dl * uu[i];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                hv[i][e] = __builtin_fmaf(exp2_hw(dl * (av[i][e] * kLog2e)), hv[i][e], dlu * bv[i][e]);
                part[i] = __builtin_fmaf(cv[i][e], hv[i][e], part[i]);
            }
            if (ok[i]) {
                if constexpr (kFull) {
                    f32x4 hw;
                    hw.x = hv[i][0]; hw.y = hv[i][1]; hw.z = hv[i][2]; hw.w = hv[i][3];
                    __builtin_nontemporal_store(hw, reinterpret_cast<f32x4 *>(p.state + rr[i] * Ns) + n0 / 4);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        if (n0 + e < Ns) p.state[rr[i] * Ns + n0 + e] = hv[i][e];
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kRpt; i++) {
        // lanes 4k..4k+3 hold one row: ((p0 + p1) + (p2 + p3)) on every lane
        float s = part[i];
        s += xor_lane<1>(s);
        s += xor_lane<2>(s);
        if (ok[i] && q == 0) {
            float y = s + dskip[i] * uu[i];
            if (p.z) y *= zz[i] * sigmoid_f32(zz[i]);
            static_cast<T *>(p.out)[rr[i]] = from_f32<T>(y);
        }
    }
}

}  // namespace

template <int R>
void launch_rows(const DecodeParams &p, bool bf16, bool full, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((p.dim + R * kRowsPerBlock - 1) / (R * kRowsPerBlock)),
                    static_cast<unsigned>(p.batch));
    if (bf16 && full)
        hipLaunchKernelGGL((ss_state_update_kernel<bf16_t, true, R>), grid, dim3(kThreads), 0, stream, p);
    else if (bf16)
        hipLaunchKernelGGL((ss_state_update_kernel<bf16_t, false, R>), grid, dim3(kThreads), 0, stream, p);
    else if (full)
        hipLaunchKernelGGL((ss_state_update_kernel<float, true, R>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((ss_state_update_kernel<float, false, R>), grid, dim3(kThreads), 0, stream, p);
}

hipError_t launch_state_update(const DecodeParams &p, bool bf16, hipStream_t stream) {
    const int64_t rows = p.batch * p.dim;
    if (rows == 0) return hipSuccess;
    // one row per 4-lane group: two or four (more bytes in flight per lane,
    // fewer waves) measured slower
    launch_rows<1>(p, bf16, p.nstate % kN == 0, stream);
    profile_mark(stream);
    return hipGetLastError();
}

}  // namespace ssk
