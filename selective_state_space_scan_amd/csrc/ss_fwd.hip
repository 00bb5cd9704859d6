// ss_fwd.hip -- forward selective scan for gfx950.
//
// Computes, for every (batch b, channel d) row,
//   h_t[n] = exp(delta_t A[d,n]) h_{t-1}[n] + delta_t B[b,n,t] u_t
//   y_t    = (sum_n C[b,n,t] h_t[n] + D[d] u_t) * silu(z_t)
// with delta_t = softplus(delta_raw_t + bias[d]) -- the selective SSM that
// the state-spaces/mamba README names under "Usage / Selective SSM".
//
// Work mapping (chosen for the MI355X execution model, not taken from any
// other GPU's kernel):
//   * one lane per (row, state index n): a 64-wide wavefront holds 4 rows x
//     16 states, one row per 16-lane DPP row; a 256-thread workgroup holds
//     16 consecutive channels of one batch entry;
//   * each lane runs the recurrence sequentially in time.  This is the
//     cheapest form of the scan in arithmetic (one exp, one multiply for
//     delta*A, one for delta*u*B and one FMA per step and state); the
//     parallelism comes from the batch x channel x state lanes, which fill
//     3-5 waves per SIMD at the Mamba layer shapes;
//   * time is staged through LDS in chunks of 32 steps with coalesced
//     16-byte global loads, prefetched one chunk ahead in registers;
//   * per-element work (softplus, delta*u, gate) is done once per element by
//     the lane whose index within the DPP row equals the step within a
//     16-step block; the scan lanes pick delta and delta*u up with a DPP row
//     broadcast instead of a memory round trip;
//   * the output sum over the 16 states goes through a padded per-wave LDS
//     transpose every 16 steps and is added in a fixed order, so a row's
//     bits do not depend on the batch size or on which other rows share the
//     workgroup.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ssk {
namespace {

constexpr int kRows = 16;             // channels per workgroup
constexpr int kT = 32;                // time steps per LDS chunk
constexpr int kThreads = 256;         // 4 wavefronts
constexpr int kPitch = kT + 4;        // padded pitch of the f32 B / C tiles
constexpr int kYBlock = kN * 16 + 16; // per-row block of the output transpose (padded)

template <typename T, int VEC>
struct Tiles {
    static constexpr int kVecPerRow = kT / VEC;
    static constexpr int kVecPerTile = 16 * kVecPerRow;
    static constexpr int kNumTiles = 5;  // B, C, u, delta, z
    static constexpr int kSlots = (kNumTiles * kVecPerTile + kThreads - 1) / kThreads;
};

struct alignas(16) Raw16 {
    uint32_t w[4];
};

template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T *__restrict__ p, int64_t t, int64_t L,
                                         bool row_ok, T (&dst)[VEC]) {
    if (row_ok && t + VEC <= L) {
        if constexpr (VEC * sizeof(T) == 16) {
            Raw16 r = *reinterpret_cast<const Raw16 *>(p + t);
            __builtin_memcpy(dst, &r, 16);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; e++) dst[e] = p[t + e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; e++) dst[e] = (row_ok && t + e < L) ? p[t + e] : T(0);
    }
}

template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void ss_fwd_kernel(FwdParams p) {
    using TL = Tiles<T, VEC>;
    __shared__ float sB[kN][kPitch];
    __shared__ float sC[kN][kPitch];
    __shared__ __attribute__((aligned(16))) T sU[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sDl[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sZ[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sO[kRows][kT];
    __shared__ __attribute__((aligned(16))) float sY[4][4 * kYBlock];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rw = lane >> 4;       // row within the wavefront (DPP row)
    const int n = lane & 15;        // state index; also the step within a 16-step block
    const int r = wave * 4 + rw;    // row within the workgroup
    const int64_t L = p.seqlen;
    const int64_t Dm = p.dim;
    const int64_t b = blockIdx.y;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x) * kRows;
    const int64_t d = d0 + r;
    const bool row_ok = d < Dm;

    const T *__restrict__ gu = static_cast<const T *>(p.u);
    const T *__restrict__ gdl = static_cast<const T *>(p.delta);
    const T *__restrict__ gz = static_cast<const T *>(p.z);
    const T *__restrict__ gB = static_cast<const T *>(p.B);
    const T *__restrict__ gC = static_cast<const T *>(p.C);
    T *__restrict__ gy = static_cast<T *>(p.out);
    const bool has_z = p.z != nullptr;

    // per-lane constants
    const float a2 = row_ok ? p.A[d * kN + n] * kLog2e : 0.0f;  // A in base-2 exponent units
    const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    const float dskip = (row_ok && p.D) ? p.D[d] : 0.0f;
    float h = (row_ok && p.h0) ? p.h0[(b * Dm + d) * kN + n] : 0.0f;

    // global -> register staging of one chunk
    T pre[TL::kSlots][VEC];
    auto fetch = [&](int64_t t0) {
#pragma unroll
        for (int k = 0; k < TL::kSlots; k++) {
            const int slot = tid + k * kThreads;
            const int tile = slot / TL::kVecPerTile;
            const int rem = slot % TL::kVecPerTile;
            const int row = rem / TL::kVecPerRow;
            const int64_t t = t0 + (rem % TL::kVecPerRow) * VEC;
            const T *base;
            bool ok;
            if (tile == 0) {
                base = gB + (b * kN + row) * L; ok = true;
            } else if (tile == 1) {
                base = gC + (b * kN + row) * L; ok = true;
            } else {
                const T *g = tile == 2 ? gu : (tile == 3 ? gdl : gz);
                ok = (tile < TL::kNumTiles) && (d0 + row < Dm) && (tile != 4 || has_z);
                base = ok ? g + (b * Dm + d0 + row) * L : gu;
            }
            load_vec<T, VEC>(base, t, L, ok, pre[k]);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int k = 0; k < TL::kSlots; k++) {
            const int slot = tid + k * kThreads;
            const int tile = slot / TL::kVecPerTile;
            if (tile >= TL::kNumTiles) continue;
            const int rem = slot % TL::kVecPerTile;
            const int row = rem / TL::kVecPerRow;
            const int col = (rem % TL::kVecPerRow) * VEC;
            if (tile < 2) {
                float *dst = tile == 0 ? &sB[row][col] : &sC[row][col];
#pragma unroll
                for (int e = 0; e < VEC; e++) dst[e] = to_f32<T>(pre[k][e]);
            } else {
                T *dst = tile == 2 ? &sU[row][col] : (tile == 3 ? &sDl[row][col] : &sZ[row][col]);
#pragma unroll
                for (int e = 0; e < VEC; e++) dst[e] = pre[k][e];
            }
        }
    };

    const int64_t nchunks = (L + kT - 1) / kT;
    if (nchunks > 0) {
        fetch(0);
        stash();
    }
    __syncthreads();

    float *ybuf = &sY[wave][0];
    for (int64_t c = 0; c < nchunks; c++) {
        const int64_t t0 = c * kT;
        if (c + 1 < nchunks) fetch(t0 + kT);

#pragma unroll
        for (int s = 0; s < kT / 16; s++) {
            // per-element work for element (r, t0 + 16 s + n)
            const int col = 16 * s + n;
            const bool t_ok = t0 + col < L;
            const float uu = to_f32<T>(sU[r][col]);
            const float zz = to_f32<T>(sZ[r][col]);
            float dl = to_f32<T>(sDl[r][col]) + bias;
            if (p.softplus) dl = softplus_f32(dl);
            if (!t_ok) dl = 0.0f;        // padding steps leave the state unchanged
            const float dlu = dl * uu;

            // 16 recurrence steps: lane (r, n) advances state entry n of row r
            float v[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&sB[n][16 * s + 4 * q]);
                const float4 c4 = *reinterpret_cast<const float4 *>(&sC[n][16 * s + 4 * q]);
                const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
                const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    float dj, duj;
                    switch (4 * q + e) {
#define SS_BCAST(J) case J: dj = row_bcast<J>(dl); duj = row_bcast<J>(dlu); break;
                        SS_BCAST(0) SS_BCAST(1) SS_BCAST(2) SS_BCAST(3)
                        SS_BCAST(4) SS_BCAST(5) SS_BCAST(6) SS_BCAST(7)
                        SS_BCAST(8) SS_BCAST(9) SS_BCAST(10) SS_BCAST(11)
                        SS_BCAST(12) SS_BCAST(13) SS_BCAST(14) SS_BCAST(15)
#undef SS_BCAST
                    }
                    const float abar = exp2_hw(dj * a2);
                    h = __builtin_fmaf(abar, h, duj * bb[e]);
                    v[4 * q + e] = cc[e] * h;
                }
            }

            // sum over the 16 states: per-wave transpose through LDS
#pragma unroll
            for (int q = 0; q < 4; q++)
                *reinterpret_cast<float4 *>(&ybuf[rw * kYBlock + n * 16 + 4 * q]) =
                    make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
            __builtin_amdgcn_wave_barrier();
            float part[16];
#pragma unroll
            for (int k = 0; k < 16; k++) part[k] = ybuf[rw * kYBlock + k * 16 + n];
            __builtin_amdgcn_wave_barrier();
            // fixed pairwise order over the state index
#pragma unroll
            for (int w = 1; w < 16; w *= 2)
#pragma unroll
                for (int k = 0; k < 16; k += 2 * w) part[k] += part[k + w];
            float y = part[0] + dskip * uu;
            if (has_z) y *= zz * sigmoid_f32(zz);
            sO[r][col] = from_f32<T>(y);
        }
        __syncthreads();

        // store the output chunk (coalesced 16-byte vectors)
        constexpr int kOutVecs = kRows * kT / VEC;
#pragma unroll
        for (int k = 0; k < (kOutVecs + kThreads - 1) / kThreads; k++) {
            const int slot = tid + k * kThreads;
            if (slot < kOutVecs) {
                const int row = slot / (kT / VEC);
                const int col = (slot % (kT / VEC)) * VEC;
                const int64_t t = t0 + col;
                if (d0 + row < Dm) {
                    T *dst = gy + (b * Dm + d0 + row) * L;
                    if (t + VEC <= L) {
                        if constexpr (VEC * sizeof(T) == 16) {
                            *reinterpret_cast<Raw16 *>(dst + t) =
                                *reinterpret_cast<const Raw16 *>(&sO[row][col]);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; e++) dst[t + e] = sO[row][col + e];
                        }
                    } else {
                        for (int e = 0; e < VEC && t + e < L; e++) dst[t + e] = sO[row][col + e];
                    }
                }
            }
        }
        if (c + 1 < nchunks) stash();
        __syncthreads();
    }

    if (p.last_state && row_ok) p.last_state[(b * Dm + d) * kN + n] = h;
}

template <typename T>
hipError_t launch_typed(const FwdParams &p, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>((p.dim + kRows - 1) / kRows), static_cast<unsigned>(p.batch));
    constexpr int kVec = 16 / sizeof(T);
    // 16-byte vectors need every row start aligned: seqlen * sizeof(T) % 16 == 0
    if ((p.seqlen * static_cast<int64_t>(sizeof(T))) % 16 == 0)
        hipLaunchKernelGGL((ss_fwd_kernel<T, kVec>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((ss_fwd_kernel<T, 1>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, bool bf16, hipStream_t stream) {
    if (p.batch == 0 || p.dim == 0) return hipSuccess;
    return bf16 ? launch_typed<bf16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssk
