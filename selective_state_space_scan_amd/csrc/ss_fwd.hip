// ss_fwd.hip -- forward selective scan for gfx950.
//
// Computes, for every (batch b, channel d) row,
//   h_t[n] = exp(delta_t A[d,n]) h_{t-1}[n] + delta_t B[b,n,t] u_t
//   y_t    = (sum_n C[b,n,t] h_t[n] + D[d] u_t) * silu(z_t)
// with delta_t = softplus(delta_raw_t + bias[d]) -- the selective SSM that
// the state-spaces/mamba README names under "Usage / Selective SSM".
//
// Work mapping (chosen for the MI355X execution model, where every wave64
// VALU instruction costs about four SIMD cycles and the LDS, shared by the
// four SIMDs of a compute unit, takes about four and a half cycles per
// wavefront read of up to 16 bytes per lane and moves about 80 bytes per
// cycle on writes):
//   * one lane per (row, state index n) for the recurrence: a 64-wide
//     wavefront holds 4 rows x 16 states, one row per 16-lane DPP row; a
//     256-thread workgroup holds 16 consecutive channels of one batch entry;
//   * each lane runs the recurrence sequentially in time: per step and state
//     one exp, a multiply for delta*A, one for (delta u)*B and one FMA --
//     the least arithmetic any form of the scan needs (the parallelism comes
//     from the batch x channel x state lanes);
//   * time runs in chunks of 64 steps.  B and C, which all channels share,
//     are staged through LDS as [state][time], prefetched a chunk ahead into
//     registers and stashed into the other of two LDS buffers, so a chunk
//     needs one barrier;
//   * per-element work (softplus, delta*u, the output, the gate) is done once
//     per element by the lane whose index in its DPP row equals the
//     element's step within a 16-step block; the scan lanes take delta and
//     delta*u from it with a DPP row broadcast folded into their multiplies;
//   * the output sum_n C h needs, at each step, a sum across the 16 lanes of
//     a row.  Every 16 steps a lane holds its 16 terms C h, and a register
//     butterfly of DPP adds over the row (levels n ^ 15 and n ^ 7 split by
//     bank mask, n ^ 2 and n ^ 1 with a select) leaves lane n the sum of
//     step n, in a fixed tree, with no LDS traffic.  Measured against an LDS
//     transpose with one FMA chain per step (fewer VALU ops, but the LDS of a
//     compute unit, shared by its four SIMDs, then became the limit) and
//     against one DPP level plus a half transpose, the register butterfly
//     was the fastest.  The backward recomputes the pre-gate output with the
//     same butterfly, so a saved and a recomputed value are the same bits;
//   * d_state above 16 runs one 16-state slice per grid z: each slice
//     writes its sums over its states as f32 partials (no D term, no gate),
//     and a combine kernel adds the slices in ascending order, adds D u and
//     applies the gate.
#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_tiles.h"

namespace ssk {
namespace {

constexpr int kT = 64;          // time steps per LDS chunk
constexpr int kPitch = kT + 4;  // f32 B / C tile pitch (conflict-free 16-byte reads)

// NW wavefronts (4 NW channels) per workgroup.  B and C (shared by all
// channels) and, for 2-byte types, the element tiles go through LDS in two
// buffers: chunk c uses buffer c & 1 while the next chunk's tiles are
// stashed into the other.
template <typename T, int NW>
struct FwdSmem {
    static constexpr uint32_t kB = 0;                          // within a buffer
    static constexpr uint32_t kC = kB + kN * kPitch * 4;
    static constexpr uint32_t kU = kC + kN * kPitch * 4;       // element tiles [row 4 NW][kT]
    static constexpr uint32_t kElem = kStageElems<T> ? 4 * NW * kT * sizeof(T) : 0;
    static constexpr uint32_t kDl = kU + kElem;
    static constexpr uint32_t kZ = kDl + kElem;
    static constexpr uint32_t kBC = kZ + kElem;                // one buffer
    static constexpr uint32_t kSize = 2 * kBC;
};

template <int J>
__device__ __forceinline__ void scan_step(float dl, float dlu, float a2, float b, float c,
                                          float &h, float &v) {
    const float abar = exp2_hw(row_bcast<J>(dl) * a2);
    h = __builtin_fmaf(abar, h, row_bcast<J>(dlu) * b);
    v = c * h;
}

// NW: wavefronts per workgroup (4 channels each).  PART: one slice of
// several (grid z); the output is the slice's f32 partial sum of C h.
template <typename T, int VEC, int NW, bool PART>
__global__ __launch_bounds__(64 * NW, VEC == 1 ? 2 : (sizeof(T) == 4 ? 3 : 4)) void ss_fwd_kernel(FwdParams p) {
    using OutT = std::conditional_t<PART, float, T>;
    using SM = FwdSmem<T, NW>;
    constexpr bool kStage = kStageElems<T>;
    constexpr int kRowsG = 4 * NW;
    constexpr int kThr = 64 * NW;
    __shared__ __attribute__((aligned(16))) char smem[SM::kSize];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rw = lane >> 4;      // row within the wavefront (DPP row)
    const int n = lane & 15;       // state index; also the step within a 16-step block
    const int r = wave * 4 + rw;   // row within the workgroup
    const int64_t L = p.seqlen;
    const int64_t Dm = p.dim;
    const int64_t b = blockIdx.y;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x) * kRowsG;
    const int64_t d = d0 + r;
    const bool row_ok = d < Dm;
    const int valid_rows = int(Dm - d0 < kRowsG ? Dm - d0 : kRowsG);
    const bool has_z = p.z != nullptr;
    // the wavefront's first row, uniform (scalar) across the wavefront
    const int64_t dw = d0 + 4 * __builtin_amdgcn_readfirstlane(wave);

    // this slice's states: s0 .. s0 + Ns - 1 of Nst; lanes n >= Ns carry
    // zero A and B, and the C^T tile zero C
    const int Nst = p.nstate;
    const int s0 = PART ? 16 * int(blockIdx.z) : 0;
    const int Ns = PART ? (Nst - s0 < kN ? Nst - s0 : kN) : Nst;
    const bool st_ok = row_ok && n < Ns;
    float a2 = st_ok ? p.A[d * Nst + s0 + n] * kLog2e : 0.0f;  // A in base-2 exponent units
    float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    float dskip = (row_ok && p.D) ? p.D[d] : 0.0f;
    float h = (st_ok && p.h0) ? p.h0[(b * Dm + d) * Nst + s0 + n] : 0.0f;

    // Inside the chunk loop time indices are 32-bit (seqlen <= 2^26), and the
    // per-row accesses address the wavefront's 4 rows from a scalar base with
    // 32-bit byte offsets (4 rows x seqlen x 4 bytes < 2^32).
    const int Ls = int(L);
    const int64_t wavebase = (b * Dm + dw) * L;
    const int rowel = rw * Ls;   // this lane's row, in elements from the wavefront's first
    const T *gu = static_cast<const T *>(p.u) + wavebase;
    const T *gdl = static_cast<const T *>(p.delta) + wavebase;
    const T *gz = has_z ? static_cast<const T *>(p.z) + wavebase : nullptr;
    const int64_t groupbase = (b * Dm + d0) * L;   // the group's first row (staged tiles)
    const T *gB = static_cast<const T *>(p.B) + (b * Nst + s0) * L;
    const T *gC = static_cast<const T *>(p.C) + (b * Nst + s0) * L;
    const bool zero_dead = Ns < kN;   // B / C rows past dstate must read as zeros
    // element t of this lane's row (0 past the end and for rows past the
    // last channel); a row's 16 lanes read 16 consecutive elements
    auto elem_at = [&](const T *g, int t) {
        return (row_ok && t < Ls)
                   ? to_f32<T>(ld_global(at_bytes(g, uint32_t(rowel + t) * uint32_t(sizeof(T)))))
                   : 0.0f;
    };
    // B and C (and the element tiles of the group's rows when staged)
    ChunkStager<T, VEC, kT, kStage ? 2 + 3 * (kRowsG / 16) : 2, kThr> st;
    st.init(
        [&](int i) -> TileSrc<T> {
            if (i == 0) return {gB, L, Ns, SM::kB, kPitch, true};
            if (i == 1) return {gC, L, Ns, SM::kC, kPitch, true};
            // element tiles in 16-row pieces; a piece with no valid row points
            // at the group's first row (it is not read)
            constexpr int kPieces = kRowsG / 16;
            const int q = (i - 2) / kPieces, j = (i - 2) % kPieces;
            const void *src = q == 0 ? p.u : q == 1 ? p.delta : p.z;
            const T *g = src ? static_cast<const T *>(src) + groupbase : nullptr;
            const uint32_t lds = q == 0 ? SM::kU : q == 1 ? SM::kDl : SM::kZ;
            const int vr = valid_rows - 16 * j;
            return {(g && vr > 0) ? g + int64_t(16 * j) * L : g, L, vr > 16 ? 16 : (vr > 0 ? vr : 0),
                    lds + uint32_t(16 * j * kT * sizeof(T)), kT, false};
        },
        tid);

    // The owned elements of a chunk (16 s + n of the lane's row) are loaded
    // during the chunk before it, once that chunk's per-element phase has
    // consumed its own, so the loads land in the same registers.
    constexpr int kE = kT / 16;
    float un[kE] = {}, dn[kE] = {}, zn[kE] = {};
    auto load_next = [&](int tc) {
        if constexpr (kStage) return;
#pragma unroll
        for (int s = 0; s < kE; s++) {
            const int t = tc + 16 * s + n;
            un[s] = elem_at(gu, t);
            dn[s] = elem_at(gdl, t);
            if (has_z) zn[s] = elem_at(gz, t);
        }
    };
    const int nchunks = int((L + kT - 1) / kT);
    if (nchunks > 0) {
        load_next(0);
        st.fetch(0, L, tid);
        st.stash(smem, zero_dead);
    }
    // Make the per-row parameter loads complete here.  Left pending into the
    // chunk loop, their first use there would be a wait on the in-order
    // memory counter that also drains the chunk prefetch.
    __asm__("" : "+v"(a2), "+v"(bias), "+v"(dskip), "+v"(h));
    __syncthreads();

    const int64_t nck = (L + kCkptSpacing - 1) / kCkptSpacing;
    const int nckS = int(nck);
    const bool save_ck = p.ckpt != nullptr;
    float *ckb = save_ck ? p.ckpt + blockIdx.z * ckpt_state_floats(p.batch, Dm, L) +
                               (b * Dm + dw) * nck * kN
                         : nullptr;
    const uint32_t ckoff = uint32_t((rw * nckS * kN + n) * 4);
    OutT *yb = (PART ? reinterpret_cast<OutT *>(p.ypart + blockIdx.z * size_t(p.batch * Dm * L))
                     : static_cast<OutT *>(p.out)) +
               wavebase;
    // the pre-gate output, saved for the backward's dz
    const bool save_yp = p.ypre && has_z;
    float *ypb = save_yp ? p.ypre + wavebase : nullptr;
    for (int c = 0; c < nchunks; c++) {
        const int t0 = c * kT;
        char *bc = smem + (c & 1) * SM::kBC;   // this chunk's staged tiles
        float(*sB)[kPitch] = reinterpret_cast<float(*)[kPitch]>(bc + SM::kB);
        float(*sC)[kPitch] = reinterpret_cast<float(*)[kPitch]>(bc + SM::kC);
        const T(*sU)[kT] = reinterpret_cast<const T(*)[kT]>(bc + SM::kU);
        const T(*sDl)[kT] = reinterpret_cast<const T(*)[kT]>(bc + SM::kDl);
        const T(*sZ)[kT] = reinterpret_cast<const T(*)[kT]>(bc + SM::kZ);
        if (c + 1 < nchunks) st.fetch(t0 + kT, L, tid);

        // per-element work: lane (r, n) owns elements 16 s + n of its row
        float dl[kE], dlu[kE], uu[kE], zz[kE];
#pragma unroll
        for (int s = 0; s < kE; s++) {
            const int col = 16 * s + n;
            float x;
            if constexpr (kStage) {
                uu[s] = to_f32<T>(sU[r][col]);
                zz[s] = has_z ? to_f32<T>(sZ[r][col]) : 0.0f;
                x = to_f32<T>(sDl[r][col]) + bias;
            } else {
                uu[s] = un[s];
                zz[s] = zn[s];
                x = dn[s] + bias;
            }
            if (p.softplus) x = softplus_f32(x);
            dl[s] = (t0 + col < Ls) ? x : 0.0f;   // padding steps leave the state unchanged
            dlu[s] = dl[s] * uu[s];
        }
        if (c + 1 < nchunks) load_next(t0 + kT);

#pragma unroll
        for (int s = 0; s < kE; s++) {
            if (save_ck && (16 * s) % kCkptSpacing == 0) {   // state entering a checkpoint block
                const int k = (t0 + 16 * s) / kCkptSpacing;
                if (row_ok && k < nckS) st_global(at_bytes(ckb, ckoff + uint32_t(k * kN * 4)), h);
            }
            float v[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 bq = *reinterpret_cast<const float4 *>(&sB[n][16 * s + 4 * q]);
                const float4 cq = *reinterpret_cast<const float4 *>(&sC[n][16 * s + 4 * q]);
                switch (q) {
#define SS_STEP4(Q)                                                                  \
    case Q:                                                                          \
        scan_step<4 * Q + 0>(dl[s], dlu[s], a2, bq.x, cq.x, h, v[4 * Q + 0]);        \
        scan_step<4 * Q + 1>(dl[s], dlu[s], a2, bq.y, cq.y, h, v[4 * Q + 1]);        \
        scan_step<4 * Q + 2>(dl[s], dlu[s], a2, bq.z, cq.z, h, v[4 * Q + 2]);        \
        scan_step<4 * Q + 3>(dl[s], dlu[s], a2, bq.w, cq.w, h, v[4 * Q + 3]);        \
        break;
                    SS_STEP4(0) SS_STEP4(1) SS_STEP4(2) SS_STEP4(3)
#undef SS_STEP4
                }
            }
            // the output of the lane's own step 16 s + n: its 16 terms summed
            // over the row by the register butterfly, + D u, the gate, the store
            const float sum = row_transpose_sum(reinterpret_cast<const float(&)[8]>(v[0]),
                                                reinterpret_cast<const float(&)[8]>(v[8]), n);
            const float ypre = PART ? sum : sum + dskip * uu[s];
            float y = ypre;
            if (has_z) y *= zz[s] * sigmoid_f32(zz[s]);
            // a row's 16 lanes store 16 consecutive outputs
            const int t = t0 + 16 * s + n;
            if (row_ok && t < Ls) {
                st_global(at_bytes(yb, uint32_t(rowel + t) * uint32_t(sizeof(OutT))), from_f32<OutT>(y));
                if (save_yp) st_global(at_bytes(ypb, uint32_t(rowel + t) * 4u), ypre);
            }
        }

        // The next chunk's tiles go to the other buffer, whose last readers
        // (the chunk before this one) are behind the previous barrier.
        if (c + 1 < nchunks) st.stash(smem + ((c + 1) & 1) * SM::kBC, zero_dead);
        __syncthreads();
    }

    if (p.last_state && st_ok) p.last_state[(b * Dm + d) * Nst + s0 + n] = h;
}

// Several slices: out = (sum of the slices' partials, ascending, + D u) *
// silu(z).  Each thread takes V consecutive elements of one row (V = 4 when
// seqlen is a multiple of 4, so the partials move as 16-byte vectors).
template <typename T, int V>
__global__ __launch_bounds__(256) void ss_fwd_combine_kernel(FwdParams p, int slices) {
    const int64_t E = p.batch * p.dim * p.seqlen;
    const int64_t e0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * V;
    if (e0 >= E) return;
    const int64_t d = (e0 / p.seqlen) % p.dim;
    const float dskip = p.D ? p.D[d] : 0.0f;
    float s[V];
    if constexpr (V == 4) {
        float4 a = *reinterpret_cast<const float4 *>(p.ypart + e0);
        for (int k = 1; k < slices; k++) {
            const float4 b = *reinterpret_cast<const float4 *>(p.ypart + k * E + e0);
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
    } else {
        s[0] = ld_global(p.ypart + e0);
        for (int k = 1; k < slices; k++) s[0] += ld_global(p.ypart + k * E + e0);
    }
    float u[V], z[V], y[V];
    if constexpr (V == 4) {
        ld4<T>(static_cast<const T *>(p.u) + e0, u);
        if (p.z) ld4<T>(static_cast<const T *>(p.z) + e0, z);
    } else {
        u[0] = to_f32<T>(ld_global(static_cast<const T *>(p.u) + e0));
        if (p.z) z[0] = to_f32<T>(ld_global(static_cast<const T *>(p.z) + e0));
    }
#pragma unroll
    for (int i = 0; i < V; i++) {
        y[i] = s[i] + dskip * u[i];
        if (p.z) y[i] *= z[i] * sigmoid_f32(z[i]);
    }
    if constexpr (V == 4) st4<T>(static_cast<T *>(p.out) + e0, y);
    else st_global(static_cast<T *>(p.out) + e0, from_f32<T>(y[0]));
}

template <typename T, int VEC, int NW, bool PART>
void launch_scan(const FwdParams &p, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((p.dim + 4 * NW - 1) / (4 * NW)),
                    static_cast<unsigned>(p.batch), static_cast<unsigned>(state_slices(p.nstate)));
    hipLaunchKernelGGL((ss_fwd_kernel<T, VEC, NW, PART>), grid, dim3(64 * NW), 0, stream, p);
}

template <typename T>
hipError_t launch_typed(const FwdParams &p, hipStream_t stream) {
    constexpr int kVec = 16 / sizeof(T);
    // 16-byte vectors need every row start aligned: seqlen * sizeof(T) % 16 == 0
    // 4 wavefronts per workgroup: 12 would cut the B / C reads by two thirds,
    // but this pass is not bound by memory, and three independent
    // workgroups per compute unit overlap their barriers and LDS phases.
    const bool vec = (p.seqlen * static_cast<int64_t>(sizeof(T))) % 16 == 0;
    const int slices = state_slices(p.nstate);
    if (slices == 1) {
        if (vec) launch_scan<T, kVec, 4, false>(p, stream);
        else launch_scan<T, 1, 4, false>(p, stream);
        profile_mark(stream);
        return hipGetLastError();
    }
    // the slices see no D term and no gate; the combine adds them
    FwdParams q = p;
    q.D = nullptr;
    q.z = nullptr;
    q.ypre = nullptr;
    if (vec) launch_scan<T, kVec, 4, true>(q, stream);
    else launch_scan<T, 1, 4, true>(q, stream);
    profile_mark(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t E = p.batch * p.dim * p.seqlen;
    if (E > 0) {
        if (p.seqlen % 4 == 0)
            hipLaunchKernelGGL((ss_fwd_combine_kernel<T, 4>), dim3(unsigned((E / 4 + 255) / 256)),
                               dim3(256), 0, stream, p, slices);
        else
            hipLaunchKernelGGL((ss_fwd_combine_kernel<T, 1>), dim3(unsigned((E + 255) / 256)),
                               dim3(256), 0, stream, p, slices);
        profile_mark(stream);
    }
    return hipGetLastError();
}

}  // namespace

size_t fwd_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int nstate) {
    const int slices = state_slices(nstate);
    if (slices == 1 || batch <= 0 || dim <= 0 || seqlen <= 0) return 0;
    return size_t(slices) * size_t(batch) * size_t(dim) * size_t(seqlen) * sizeof(float);
}

hipError_t launch_fwd(const FwdParams &p, bool bf16, hipStream_t stream) {
    if (p.batch == 0 || p.dim == 0) return hipSuccess;
    return bf16 ? launch_typed<bf16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssk
