// ss_fwd.hip -- forward selective scan for gfx950.
//
// Computes, for every (batch b, channel d) row,
//   h_t[n] = exp(delta_t A[d,n]) h_{t-1}[n] + delta_t B[b,n,t] u_t
//   y_t    = (sum_n C[b,n,t] h_t[n] + D[d] u_t) * silu(z_t)
// with delta_t = softplus(delta_raw_t + bias[d]) -- the selective SSM that
// the state-spaces/mamba README names under "Usage / Selective SSM".
//
// Work mapping (chosen for the MI355X execution model):
//   * one lane per (row, state index n): a 64-wide wavefront holds 4 rows x
//     16 states, one row per 16-lane DPP row; a 256-thread workgroup holds
//     16 consecutive channels of one batch entry;
//   * each lane runs the recurrence sequentially in time.  This is the
//     cheapest form of the scan in arithmetic (per step and state: one
//     exp, a multiply for delta*A, one for delta*u*B and one FMA); the
//     parallelism comes from the batch x channel x state lanes, which fill
//     3-5 waves per SIMD at the Mamba layer shapes;
//   * time is staged through LDS in chunks of 64 steps with coalesced
//     16-byte loads, prefetched one chunk ahead into registers;
//   * per-element work (softplus, delta*u, gate) is done once per element by
//     the lane whose index in its DPP row equals the element's step within a
//     16-step block; the scan lanes take delta and delta*u from it with a DPP
//     row broadcast folded into their multiplies;
//   * the output's sum over the 16 states goes through a per-wave LDS
//     transpose every 16 steps, padded so that neither the 16-byte writes
//     nor the 4-byte reads hit the same bank twice, and is added in a fixed
//     order -- a row's bits do not depend on the batch size or on the other
//     rows of its workgroup.
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_tiles.h"

namespace ssk {
namespace {

constexpr int kRows = 16;       // channels per workgroup
constexpr int kT = 64;          // time steps per LDS chunk
constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kPitch = kT + 4;  // f32 B / C tile pitch (conflict-free 16-byte reads)
constexpr int kYN = 20;         // transpose: floats per state entry (16 + 4 pad)
constexpr int kYRow = 16 * kYN + 16;  // transpose: floats per row (row offset = 16 banks)

template <typename T>
struct FwdSmem {
    static constexpr uint32_t kB = 0;
    static constexpr uint32_t kC = kB + kN * kPitch * 4;
    static constexpr uint32_t kU = kC + kN * kPitch * 4;                  // union start
    static constexpr uint32_t kDl = kU + kRows * kT * sizeof(T);
    static constexpr uint32_t kZ = kDl + kRows * kT * sizeof(T);
    static constexpr uint32_t kY = kU;                                    // aliases u / delta / z
    static constexpr uint32_t kRawEnd = kZ + kRows * kT * sizeof(T);
    static constexpr uint32_t kYEnd = kY + 4 * 4 * kYRow * 4;
    static constexpr uint32_t kSize = kRawEnd > kYEnd ? kRawEnd : kYEnd;
};

template <int J>
__device__ __forceinline__ void scan_step(float dl, float dlu, float a2, float b, float c,
                                          float &h, float &v) {
    const float abar = exp2_hw(row_bcast<J>(dl) * a2);
    h = __builtin_fmaf(abar, h, row_bcast<J>(dlu) * b);
    v = c * h;
}

template <typename T, int VEC>
__global__ __launch_bounds__(kThreads, VEC == 1 ? 2 : (sizeof(T) == 4 ? 3 : 4)) void ss_fwd_kernel(FwdParams p) {
    using SM = FwdSmem<T>;
    __shared__ __attribute__((aligned(16))) char smem[SM::kSize];
    float(*sB)[kPitch] = reinterpret_cast<float(*)[kPitch]>(smem + SM::kB);
    float(*sC)[kPitch] = reinterpret_cast<float(*)[kPitch]>(smem + SM::kC);
    T(*sU)[kT] = reinterpret_cast<T(*)[kT]>(smem + SM::kU);
    T(*sDl)[kT] = reinterpret_cast<T(*)[kT]>(smem + SM::kDl);
    T(*sZ)[kT] = reinterpret_cast<T(*)[kT]>(smem + SM::kZ);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rw = lane >> 4;      // row within the wavefront (DPP row)
    const int n = lane & 15;       // state index; also the step within a 16-step block
    const int r = wave * 4 + rw;   // row within the workgroup
    const int64_t L = p.seqlen;
    const int64_t Dm = p.dim;
    const int64_t b = blockIdx.y;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x) * kRows;
    const int64_t d = d0 + r;
    const bool row_ok = d < Dm;
    const int valid_rows = static_cast<int>(Dm - d0 < kRows ? Dm - d0 : kRows);
    const bool has_z = p.z != nullptr;

    float a2 = row_ok ? p.A[d * kN + n] * kLog2e : 0.0f;  // A in base-2 exponent units
    float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    float dskip = (row_ok && p.D) ? p.D[d] : 0.0f;
    float h = (row_ok && p.h0) ? p.h0[(b * Dm + d) * kN + n] : 0.0f;

    const T *gu = static_cast<const T *>(p.u) + (b * Dm + d0) * L;
    const T *gdl = static_cast<const T *>(p.delta) + (b * Dm + d0) * L;
    const T *gz = has_z ? static_cast<const T *>(p.z) + (b * Dm + d0) * L : nullptr;
    const T *gB = static_cast<const T *>(p.B) + b * kN * L;
    const T *gC = static_cast<const T *>(p.C) + b * kN * L;
    ChunkStager<T, VEC, kT, 5, kThreads> st;
    st.init(
        [&](int i) -> TileSrc<T> {
            switch (i) {
                case 0: return {gB, L, kN, SM::kB, kPitch, true};
                case 1: return {gC, L, kN, SM::kC, kPitch, true};
                case 2: return {gu, L, valid_rows, SM::kU, kT, false};
                case 3: return {gdl, L, valid_rows, SM::kDl, kT, false};
                default: return {gz, L, valid_rows, SM::kZ, kT, false};
            }
        },
        tid);

    const int64_t nchunks = (L + kT - 1) / kT;
    if (nchunks > 0) {
        st.fetch(0, L, tid);
        st.stash(smem);
    }
    // Make the per-row parameter loads complete here.  Left pending into the
    // chunk loop, their first use there would be a wait on the in-order
    // memory counter that also drains the chunk prefetch.
    __asm__("" : "+v"(a2), "+v"(bias), "+v"(dskip), "+v"(h));
    __syncthreads();

    // Inside the chunk loop time indices are 32-bit (seqlen <= 2^26), and the
    // stores address the group's 16 rows from a scalar base with 32-bit byte
    // offsets (16 rows x seqlen x 4 bytes < 2^32).
    const int Ls = int(L);
    const int64_t nck = (L + kCkptSpacing - 1) / kCkptSpacing;
    const int nckS = int(nck);
    const bool save_ck = p.ckpt != nullptr;
    float *ckb = save_ck ? p.ckpt + (b * Dm + d0) * nck * kN : nullptr;
    const uint32_t ckoff = uint32_t((r * nckS * kN + n) * 4);
    float *ybuf = reinterpret_cast<float *>(smem + SM::kY) + wave * 4 * kYRow + rw * kYRow;
    T *yb = static_cast<T *>(p.out) + (b * Dm + d0) * L;
    // the pre-gate output, saved for the backward's dz
    const bool save_yp = p.ypre && has_z;
    float *ypb = save_yp ? p.ypre + (b * Dm + d0) * L : nullptr;
    const int rowel = r * Ls;   // this lane's row, in elements from the group's first
    for (int c = 0; c < int(nchunks); c++) {
        const int t0 = c * kT;
        if (c + 1 < nchunks) st.fetch(t0 + kT, L, tid);

        // per-element work: lane (r, n) owns elements 16 s + n of its row
        float dl[kT / 16], dlu[kT / 16], uu[kT / 16], zz[kT / 16];
#pragma unroll
        for (int s = 0; s < kT / 16; s++) {
            const int col = 16 * s + n;
            uu[s] = to_f32<T>(sU[r][col]);
            zz[s] = to_f32<T>(sZ[r][col]);
            float x = to_f32<T>(sDl[r][col]) + bias;
            if (p.softplus) x = softplus_f32(x);
            dl[s] = (t0 + col < Ls) ? x : 0.0f;   // padding steps leave the state unchanged
            dlu[s] = dl[s] * uu[s];
        }
        __syncthreads();  // the transpose region aliases u / delta / z

        // Output sums over the 16 states go through this wave's LDS region:
        // block s writes its per-state terms four steps at a time; their
        // transposed reads are issued at the start of block s + 1 and summed
        // at its end, so the LDS round trip overlaps the next 16 steps.
        float part[16];
        auto finish = [&](int s) {
            // in the order of the backward's register butterfly, so the
            // saved pre-gate output matches its recomputation bit for bit
            const float ypre = row_tree_sum(part) + dskip * uu[s];
            float y = ypre;
            if (has_z) y *= zz[s] * sigmoid_f32(zz[s]);
            // a row's 16 lanes store 16 consecutive outputs
            const int t = t0 + 16 * s + n;
            if (row_ok && t < Ls) {
                st_global(at_bytes(yb, uint32_t(rowel + t) * uint32_t(sizeof(T))), from_f32<T>(y));
                if (save_yp) st_global(at_bytes(ypb, uint32_t(rowel + t) * 4u), ypre);
            }
        };
#pragma unroll
        for (int s = 0; s < kT / 16; s++) {
            if (save_ck && (16 * s) % kCkptSpacing == 0) {   // state entering a checkpoint chunk
                const int k = (t0 + 16 * s) / kCkptSpacing;
                if (row_ok && k < nckS) st_global(at_bytes(ckb, ckoff + uint32_t(k * kN * 4)), h);
            }
            float4 bq[4], cq[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                bq[q] = *reinterpret_cast<const float4 *>(&sB[n][16 * s + 4 * q]);
                cq[q] = *reinterpret_cast<const float4 *>(&sC[n][16 * s + 4 * q]);
            }
            if (s > 0) {
#pragma unroll
                for (int k = 0; k < 16; k++) part[k] = ybuf[k * kYN + n];
            }
#pragma unroll
            for (int q = 0; q < 4; q++) {
                float v[4];
                switch (q) {
#define SS_STEP4(Q)                                                                  \
    case Q:                                                                          \
        scan_step<4 * Q + 0>(dl[s], dlu[s], a2, bq[Q].x, cq[Q].x, h, v[0]);          \
        scan_step<4 * Q + 1>(dl[s], dlu[s], a2, bq[Q].y, cq[Q].y, h, v[1]);          \
        scan_step<4 * Q + 2>(dl[s], dlu[s], a2, bq[Q].z, cq[Q].z, h, v[2]);          \
        scan_step<4 * Q + 3>(dl[s], dlu[s], a2, bq[Q].w, cq[Q].w, h, v[3]);          \
        break;
                    SS_STEP4(0) SS_STEP4(1) SS_STEP4(2) SS_STEP4(3)
#undef SS_STEP4
                }
                // in-order LDS: this write lands after the reads issued above
                *reinterpret_cast<float4 *>(&ybuf[n * kYN + 4 * q]) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
            if (s > 0) finish(s - 1);
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < 16; k++) part[k] = ybuf[k * kYN + n];
        finish(kT / 16 - 1);
        __syncthreads();

        if (c + 1 < nchunks) st.stash(smem);
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
    profile_mark(stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, bool bf16, hipStream_t stream) {
    if (p.batch == 0 || p.dim == 0) return hipSuccess;
    return bf16 ? launch_typed<bf16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssk
