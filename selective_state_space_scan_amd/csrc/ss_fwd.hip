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
//   * d_state above 16 is cut into 16-state slices.  Up to 64 states a lane
//     runs the same state index of every slice of its row (states n, 16 + n,
//     ...), and a step's terms C h are added over the slices in the lane, in
//     ascending order, before the one butterfly: no partials leave the chip.
//     Above 64 states one slice runs per grid z, each writing its sums over
//     its states as f32 partials (no D term, no gate), and a combine kernel
//     adds the slices in ascending order, adds D u and applies the gate.
#include <type_traits>

#include "ss_conv_lane.h"
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_tiles.h"

namespace ssk {
namespace {

constexpr int kT = 64;          // time steps per LDS chunk
constexpr int kPitch = kT + 4;  // f32 B / C tile pitch (conflict-free 16-byte reads)

// NW wavefronts (4 NW channels) per workgroup, S 16-state slices per lane.
// B and C (shared by all channels; S tiles of 16 states each) and, for
// 2-byte types, the element tiles go through LDS in two buffers: chunk c
// uses buffer c & 1 while the next chunk's tiles are stashed into the
// other.  With three or four slices a chunk is 32 steps, so that three
// workgroups still fit a compute unit's LDS.
template <typename T, int NW, int S = 1>
struct FwdSmem {
    static constexpr int kTc = S <= 2 ? kT : 32;              // steps per chunk
    static constexpr int kPitchC = kTc + 4;
    static constexpr uint32_t kB = 0;                          // within a buffer
    static constexpr uint32_t kC = kB + S * kN * kPitchC * 4;
    static constexpr uint32_t kU = kC + S * kN * kPitchC * 4;  // element tiles [row 4 NW][kTc]
    static constexpr uint32_t kElem = kStageElems<T> ? 4 * NW * kTc * sizeof(T) : 0;
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
// the same step of a further slice of the lane's row: its term C h is added
// to the step's running sum over the slices
template <int J>
__device__ __forceinline__ void scan_step_acc(float dl, float dlu, float a2, float b, float c,
                                              float &h, float &v) {
    const float abar = exp2_hw(row_bcast<J>(dl) * a2);
    h = __builtin_fmaf(abar, h, row_bcast<J>(dlu) * b);
    v = __builtin_fmaf(c, h, v);
}

// Where segment j's summary (end state from zero, then total decay) of
// slice sl, batch entry b, row d, state n lives.
__device__ __forceinline__ size_t summ_index(const FwdParams &p, int sl, int j, int64_t b,
                                             int64_t d, int n) {
    return seg_summ_index(p.nseg, p.batch, p.dim, sl, j, b, d, n);
}
__device__ __forceinline__ size_t summ_decay_offset(const FwdParams &p) {
    return seg_summ_half(p.nstate, p.nseg, p.batch, p.dim);
}

// The summary pass of a segmented scan: every segment but the last from a
// zero state, the recurrence only, writing the segment's end state and its
// total decay exp(A sum delta).  16 channels (4 wavefronts) per workgroup,
// B, u and delta staged through LDS in 64-step chunks, two buffers (the
// next chunk is stashed into the other while this one is read, one barrier
// per chunk); grid z holds (slice, segment < nseg - 1).
constexpr int kTS = 64;
constexpr int kPitchS = kTS + 4;

template <typename T>
struct SumSmem {
    static constexpr uint32_t kB = 0;
    static constexpr uint32_t kU = kB + kN * kPitchS * 4;
    static constexpr uint32_t kDl = kU + 16 * kTS * sizeof(T);
    static constexpr uint32_t kSize = kDl + 16 * kTS * sizeof(T);
};

template <int J>
__device__ __forceinline__ float state_step(float dl, float dlu, float a2, float b, float h) {
    return __builtin_fmaf(exp2_hw(row_bcast<J>(dl) * a2), h, row_bcast<J>(dlu) * b);
}

template <typename T, int VEC, int CONV = 0>
__global__ __launch_bounds__(256) void ss_fwd_summary_kernel(FwdParams p) {
    using SM = SumSmem<T>;
    __shared__ __attribute__((aligned(16))) char smem[2 * SM::kSize];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, r = wave * 4 + (lane >> 4);
    const int64_t L = p.seqlen, Dm = p.dim, b = blockIdx.y;
    const int64_t d0 = int64_t(blockIdx.x) * 16, d = d0 + r;
    const bool row_ok = d < Dm;
    const int valid_rows = int(Dm - d0 < 16 ? Dm - d0 : 16);
    const int nz = p.nseg - 1;
    const int slice = int(blockIdx.z) / nz, seg = int(blockIdx.z) % nz;
    const int Nst = p.nstate, s0 = 16 * slice;
    const int Ns = Nst - s0 < kN ? Nst - s0 : kN;
    const bool st_ok = row_ok && n < Ns;
    const float a2 = st_ok ? p.A[d * Nst + s0 + n] * kLog2e : 0.0f;
    const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    const T *gB = static_cast<const T *>(p.B) + (b * Nst + s0) * L;
    const T *gu = static_cast<const T *>(p.u) + (b * Dm + d0) * L;
    const T *gdl = static_cast<const T *>(p.delta) + (b * Dm + d0) * L;
    ChunkStager<T, VEC, kTS, 3, 256> st;
    st.init(
        [&](int i) -> TileSrc<T> {
            switch (i) {
                case 0: return {gB, L, Ns, SM::kB, kPitchS, true};
                case 1: return {gu, L, valid_rows, SM::kU, kTS, false};
                default: return {gdl, L, valid_rows, SM::kDl, kTS, false};
            }
        },
        tid);
    // a segment before the last: whole 64-step chunks
    const int64_t tbeg = int64_t(seg) * p.seg_len;
    const int nchunk = p.seg_len / kTS;
    float h = 0.0f, dlsum = 0.0f;
    // fused convolution: the staged u tile holds its input x
    ConvLane cv{};
    float xprev = 0.0f;
    if constexpr (CONV != 0) {
        cv = conv_lane(p, d, row_ok);
        xprev = conv_prev<T>(p, b, d, row_ok, tbeg, n);
    }
    st.fetch(tbeg, L, tid);
    st.stash(smem, Ns < kN);
    __syncthreads();
    for (int c = 0; c < nchunk; c++) {
        const int64_t t0 = tbeg + int64_t(c) * kTS;
        char *buf = smem + (c & 1) * SM::kSize;
        float(*sB)[kPitchS] = reinterpret_cast<float(*)[kPitchS]>(buf + SM::kB);
        const T(*sU)[kTS] = reinterpret_cast<const T(*)[kTS]>(buf + SM::kU);
        const T(*sDl)[kTS] = reinterpret_cast<const T(*)[kTS]>(buf + SM::kDl);
        if (c + 1 < nchunk) st.fetch(t0 + kTS, L, tid);
        float dl[kTS / 16], dlu[kTS / 16];
#pragma unroll
        for (int s = 0; s < kTS / 16; s++) {
            const int col = 16 * s + n;
            float x = to_f32<T>(sDl[r][col]) + bias;
            if (p.softplus) x = softplus_f32(x);
            dl[s] = row_ok ? x : 0.0f;
            float uv = to_f32<T>(sU[r][col]);
            if constexpr (CONV != 0) {
                const float xin = uv;
                uv = row_ok ? conv_u<T, (CONV > 0 ? CONV : 0)>(cv, xin, xprev) : 0.0f;
                xprev = xin;
            }
            dlu[s] = dl[s] * uv;
            dlsum += dl[s];
        }
#pragma unroll
        for (int s = 0; s < kTS / 16; s++) {
            const float dls = dl[s], dlus = dlu[s];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&sB[n][16 * s + 4 * q]);
                switch (q) {
#define SS_SSTEP4(Q)                                                       \
    case Q:                                                                \
        h = state_step<4 * Q + 0>(dls, dlus, a2, b4.x, h);                 \
        h = state_step<4 * Q + 1>(dls, dlus, a2, b4.y, h);                 \
        h = state_step<4 * Q + 2>(dls, dlus, a2, b4.z, h);                 \
        h = state_step<4 * Q + 3>(dls, dlus, a2, b4.w, h);                 \
        break;
                    SS_SSTEP4(0) SS_SSTEP4(1) SS_SSTEP4(2) SS_SSTEP4(3)
#undef SS_SSTEP4
                }
            }
        }
        // the state is complete before the barrier: left free, the
        // register-only recurrence sinks past it into the next iteration,
        // with every broadcast of the chunk live across the loop edge
        __asm__ volatile("" : "+v"(h));
        // the other buffer's last readers (the chunk before) are behind the
        // previous barrier
        if (c + 1 < nchunk) st.stash(smem + ((c + 1) & 1) * SM::kSize, Ns < kN);
        __syncthreads();
    }
    // the decay exp(A sum delta) from the row's delta sum, formed in one
    // fixed tree over its 16 lanes (every lane gets the same bits)
    const float tot = row_sum16(dlsum);
    if (row_ok) {
        const size_t i = summ_index(p, slice, seg, b, d, n);
        p.summ[i] = h;
        p.summ[summ_decay_offset(p) + i] = exp2_hw(a2 * tot);
    }
}

// NW: wavefronts per workgroup (4 channels each).  PART: one slice of
// several; the output is the slice's f32 partial sum of C h.  S > 1: each
// lane runs the same state index of S slices (states n, 16 + n, ...); the
// terms C h of a step are added over the slices in the lane, in ascending
// order, before the sum over the row's 16 lanes.  Grid z holds (slice, time
// segment); with S > 1 it holds the segment only.
// CONV: 0 no convolution; 4 the fused convolution of width 4; -1 of the
// width p.conv_width
template <typename T, int VEC, int NW, bool PART, int S = 1, int CONV = 0>
__global__ __launch_bounds__(64 * NW, VEC == 1 ? 2 : (sizeof(T) == 4 ? 3 : 4)) void ss_fwd_kernel(FwdParams p) {
    static_assert(S >= 1 && !(PART && S > 1), "slices run either in the lane or one per grid z");
    static_assert(!(PART && CONV), "the fused convolution runs with the slices in the lane");
    using OutT = std::conditional_t<PART, float, T>;
    using SM = FwdSmem<T, NW, S>;
    constexpr int kT = SM::kTc;          // steps per chunk
    constexpr int kPitch = SM::kPitchC;
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

    // grid z: (slice, segment).  Lane slice k holds states s0 + 16 k + n;
    // states past dstate carry zero A, B and C
    const int slice = int(blockIdx.z) / p.nseg, seg = int(blockIdx.z) % p.nseg;
    const int Nst = p.nstate;
    const int s0 = PART ? 16 * slice : 0;
    auto slice_states = [&](int k) {   // valid states of lane slice k
        const int first = s0 + 16 * k;
        return (PART || S > 1) ? (Nst - first < kN ? Nst - first : kN) : Nst;
    };
    float a2[S], h[S];   // A in base-2 exponent units; the state
#pragma unroll
    for (int k = 0; k < S; k++) {
        const bool ok = row_ok && n < slice_states(k);
        a2[k] = ok ? p.A[d * Nst + s0 + 16 * k + n] * kLog2e : 0.0f;
        h[k] = (ok && p.h0) ? p.h0[(b * Dm + d) * Nst + s0 + 16 * k + n] : 0.0f;
    }
    float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    float dskip = (row_ok && p.D) ? p.D[d] : 0.0f;
    if (seg > 0 && row_ok) {
        // the state entering this segment: the segments before it, each a
        // (decay, end state from zero) pair, applied in ascending order
        const float *sh = p.summ, *sd = p.summ + summ_decay_offset(p);
#pragma unroll
        for (int k = 0; k < S; k++) {
            for (int j = 0; j < seg; j++) {
                const size_t i = summ_index(p, PART ? slice : k, j, b, d, n);
                h[k] = __builtin_fmaf(sd[i], h[k], sh[i]);
            }
        }
    }
    // this segment's steps and 64-step chunks
    const int64_t tbeg = int64_t(seg) * p.seg_len;
    const int64_t tend = tbeg + p.seg_len < p.seqlen ? tbeg + p.seg_len : p.seqlen;

    // Inside the chunk loop time indices are 32-bit (seqlen <= 2^26), and the
    // per-row accesses address the wavefront's 4 rows from a scalar base with
    // 32-bit byte offsets (4 rows x seqlen x 4 bytes < 2^32).
    // Lanes of rows past the last channel address the last channel's row
    // instead: their loads stay in bounds (the values are not used) and
    // their stores are skipped, so the loads of whole chunks need no guard.
    const int Ls = int(L);
    const int64_t dwc = dw < Dm ? dw : Dm - 1;
    const int rwc = int((row_ok ? d : Dm - 1) - dwc);
    const int64_t wavebase = (b * Dm + dwc) * L;
    const int rowel = rwc * Ls;   // this lane's row, in elements from the wavefront's first
    const T *gu = static_cast<const T *>(p.u) + wavebase;
    const T *gdl = static_cast<const T *>(p.delta) + wavebase;
    const T *gz = has_z ? static_cast<const T *>(p.z) + wavebase : nullptr;
    const int64_t groupbase = (b * Dm + d0) * L;   // the group's first row (staged tiles)
    const T *gB = static_cast<const T *>(p.B) + (b * Nst + s0) * L;
    const T *gC = static_cast<const T *>(p.C) + (b * Nst + s0) * L;
    const bool zero_dead = slice_states(S - 1) < kN;   // B / C rows past dstate must read as zeros
    // element t of this lane's row (0 past the end and for rows past the
    // last channel); a row's 16 lanes read 16 consecutive elements
    auto elem_at = [&](const T *g, int t) {
        return (row_ok && t < Ls)
                   ? to_f32<T>(ld_global(at_bytes(g, uint32_t(rowel + t) * uint32_t(sizeof(T)))))
                   : 0.0f;
    };
    // B and C (and the element tiles of the group's rows when staged)
    ChunkStager<T, VEC, kT, kStage ? 2 * S + 3 * (kRowsG / 16) : 2 * S, kThr> st;
    st.init(
        [&](int i) -> TileSrc<T> {
            // B of slices 0 .. S - 1, then C of slices 0 .. S - 1
            if (i < S) return {gB + int64_t(16 * i) * L, L, slice_states(i),
                               SM::kB + uint32_t(i * kN * kPitch * 4), kPitch, true};
            if (i < 2 * S) return {gC + int64_t(16 * (i - S)) * L, L, slice_states(i - S),
                                   SM::kC + uint32_t((i - S) * kN * kPitch * 4), kPitch, true};
            // element tiles in 16-row pieces; a piece with no valid row points
            // at the group's first row (it is not read)
            constexpr int kPieces = kRowsG / 16;
            const int q = (i - 2 * S) / kPieces, j = (i - 2 * S) % kPieces;
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
    // whole: every step of the chunk is before the sequence's end, and the
    // loads go unguarded (the row is taken care of by the clamped row above)
    auto elem_whole = [&](const T *g, int t) {
        return to_f32<T>(ld_global(at_bytes(g, uint32_t(rowel + t) * uint32_t(sizeof(T)))));
    };
    auto load_next = [&](int tc, bool whole) {
        if constexpr (kStage) return;
#pragma unroll
        for (int s = 0; s < kE; s++) {
            const int t = tc + 16 * s + n;
            un[s] = whole ? elem_whole(gu, t) : elem_at(gu, t);
            dn[s] = whole ? elem_whole(gdl, t) : elem_at(gdl, t);
            if (has_z) zn[s] = whole ? elem_whole(gz, t) : elem_at(gz, t);
        }
    };
    const int cbeg = int(tbeg / kT);
    const int cend = int((tend + kT - 1) / kT);
    if (cend > cbeg) {
        load_next(cbeg * kT, false);
        st.fetch(int64_t(cbeg) * kT, L, tid);
        st.stash(smem, zero_dead);
    }
    // fused convolution: u holds its input x; the lane's input one block
    // before the segment's first step
    ConvLane cv{};
    float xprev = 0.0f;
    if constexpr (CONV != 0) {
        cv = conv_lane(p, d, row_ok);
        xprev = conv_prev<T>(p, b, d, row_ok, tbeg, n);
        __asm__("" : "+v"(xprev), "+v"(cv.b), "+v"(cv.wl[0]), "+v"(cv.wl[1]), "+v"(cv.wl[2]),
                "+v"(cv.wl[3]));
    }
    // Make the per-row parameter loads complete here.  Left pending into the
    // chunk loop, their first use there would be a wait on the in-order
    // memory counter that also drains the chunk prefetch.
    __asm__("" : "+v"(bias), "+v"(dskip));
#pragma unroll
    for (int k = 0; k < S; k++) __asm__("" : "+v"(a2[k]), "+v"(h[k]));
    __syncthreads();

    const int64_t nck = (L + kCkptSpacing - 1) / kCkptSpacing;
    const int nckS = int(nck);
    const bool save_ck = p.ckpt != nullptr;
    // block states of lane slice k: k ckpt_state_floats further on
    const size_t ck_slice = ckpt_state_floats(p.batch, Dm, L);
    float *ckb = save_ck ? p.ckpt + slice * ck_slice + (b * Dm + dw) * nck * kN : nullptr;
    const uint32_t ckoff = uint32_t((rw * nckS * kN + n) * 4);
    OutT *yb = (PART ? reinterpret_cast<OutT *>(p.ypart + slice * size_t(p.batch * Dm * L))
                     : static_cast<OutT *>(p.out)) +
               wavebase;
    // the pre-gate output, saved for the backward's dz
    const bool save_yp = p.ypre && has_z;
    float *ypb = save_yp ? p.ypre + wavebase : nullptr;
    for (int c = cbeg; c < cend; c++) {
        const int t0 = c * kT;
        const bool more = c + 1 < cend;
        char *bc = smem + ((c - cbeg) & 1) * SM::kBC;   // this chunk's staged tiles
        float(*sB)[kPitch] = reinterpret_cast<float(*)[kPitch]>(bc + SM::kB);
        float(*sC)[kPitch] = reinterpret_cast<float(*)[kPitch]>(bc + SM::kC);
        const T(*sU)[kT] = reinterpret_cast<const T(*)[kT]>(bc + SM::kU);
        const T(*sDl)[kT] = reinterpret_cast<const T(*)[kT]>(bc + SM::kDl);
        const T(*sZ)[kT] = reinterpret_cast<const T(*)[kT]>(bc + SM::kZ);
        if (more) st.fetch(t0 + kT, L, tid);

        // per-element work: lane (r, n) owns elements 16 s + n of its row
        float dl[kE], dlu[kE], uu[kE], zz[kE];
        // the staged elements, all read before any is used (a read behind a
        // branch would wait for each one in turn); z's tile is read even
        // without z (its value is then not used)
        T su[kE], sd[kE], sz[kE];
        if constexpr (kStage) {
#pragma unroll
            for (int s = 0; s < kE; s++) {
                su[s] = sU[r][16 * s + n];
                sd[s] = sDl[r][16 * s + n];
                sz[s] = sZ[r][16 * s + n];
            }
        }
#pragma unroll
        for (int s = 0; s < kE; s++) {
            const int col = 16 * s + n;
            float x;
            if constexpr (kStage) {
                uu[s] = to_f32<T>(su[s]);
                zz[s] = has_z ? to_f32<T>(sz[s]) : 0.0f;
                x = to_f32<T>(sd[s]) + bias;
            } else {
                uu[s] = un[s];
                zz[s] = zn[s];
                x = dn[s] + bias;
            }
            if constexpr (CONV != 0) {   // uu held the convolution's input
                const float xin = uu[s];
                uu[s] = row_ok ? conv_u<T, (CONV > 0 ? CONV : 0)>(cv, xin, xprev) : 0.0f;
                xprev = xin;
            }
            if (p.softplus) x = softplus_f32(x);
            dl[s] = (t0 + col < Ls) ? x : 0.0f;   // padding steps leave the state unchanged
            dlu[s] = row_ok ? dl[s] * uu[s] : 0.0f;
        }
        if (more) {
            if (t0 + 2 * kT <= Ls) load_next(t0 + kT, true);
            else load_next(t0 + kT, false);
        }

#pragma unroll
        for (int s = 0; s < kE; s++) {
            if (save_ck && (16 * s) % kCkptSpacing == 0) {   // state entering a checkpoint block
                const int k = (t0 + 16 * s) / kCkptSpacing;
                if (row_ok && k < nckS) {
#pragma unroll
                    for (int i = 0; i < S; i++)
                        st_global(at_bytes(ckb + i * ck_slice, ckoff + uint32_t(k * kN * 4)), h[i]);
                }
            }
            float v[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
#pragma unroll
                for (int i = 0; i < S; i++) {
                    // slice i's B and C rows: 16 i + n
                    const float4 bq = *reinterpret_cast<const float4 *>(&sB[16 * i + n][16 * s + 4 * q]);
                    const float4 cq = *reinterpret_cast<const float4 *>(&sC[16 * i + n][16 * s + 4 * q]);
                    if (i == 0) {
                        switch (q) {
#define SS_STEP4(Q)                                                                        \
    case Q:                                                                                \
        scan_step<4 * Q + 0>(dl[s], dlu[s], a2[0], bq.x, cq.x, h[0], v[4 * Q + 0]);        \
        scan_step<4 * Q + 1>(dl[s], dlu[s], a2[0], bq.y, cq.y, h[0], v[4 * Q + 1]);        \
        scan_step<4 * Q + 2>(dl[s], dlu[s], a2[0], bq.z, cq.z, h[0], v[4 * Q + 2]);        \
        scan_step<4 * Q + 3>(dl[s], dlu[s], a2[0], bq.w, cq.w, h[0], v[4 * Q + 3]);        \
        break;
                            SS_STEP4(0) SS_STEP4(1) SS_STEP4(2) SS_STEP4(3)
#undef SS_STEP4
                        }
                    } else {
                        switch (q) {
#define SS_STEP4(Q)                                                                            \
    case Q:                                                                                    \
        scan_step_acc<4 * Q + 0>(dl[s], dlu[s], a2[i], bq.x, cq.x, h[i], v[4 * Q + 0]);        \
        scan_step_acc<4 * Q + 1>(dl[s], dlu[s], a2[i], bq.y, cq.y, h[i], v[4 * Q + 1]);        \
        scan_step_acc<4 * Q + 2>(dl[s], dlu[s], a2[i], bq.z, cq.z, h[i], v[4 * Q + 2]);        \
        scan_step_acc<4 * Q + 3>(dl[s], dlu[s], a2[i], bq.w, cq.w, h[i], v[4 * Q + 3]);        \
        break;
                            SS_STEP4(0) SS_STEP4(1) SS_STEP4(2) SS_STEP4(3)
#undef SS_STEP4
                        }
                    }
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
            // The next chunk's tiles go to the other buffer, whose last
            // readers (the chunk before this one) are behind the previous
            // barrier.  They go before the last block's outputs: the wait
            // for the staged loads would otherwise also wait for the write
            // acknowledgments of those stores.
            if (s == kE - 1 && more) st.stash(smem + ((c + 1 - cbeg) & 1) * SM::kBC, zero_dead);
            const int t = t0 + 16 * s + n;
            if (row_ok && t < Ls) {
                // (no out: the backward builds its record with this kernel)
                if (p.out) st_global(at_bytes(yb, uint32_t(rowel + t) * uint32_t(sizeof(OutT))), from_f32<OutT>(y));
                if (save_yp) st_global(at_bytes(ypb, uint32_t(rowel + t) * 4u), ypre);
            }
        }
        __syncthreads();
    }

    if (CONV != 0 && p.conv_final && row_ok && seg == p.nseg - 1 && n < p.conv_width - 1) {
        // the convolution's final window: the row's last H inputs
        const int H = p.conv_width - 1;
        p.conv_final[(b * Dm + d) * H + n] = conv_prev<T>(p, b, d, row_ok, L - H + 16, n);
    }
    if (p.last_state && row_ok && seg == p.nseg - 1) {
#pragma unroll
        for (int k = 0; k < S; k++)
            if (n < slice_states(k)) p.last_state[(b * Dm + d) * Nst + s0 + 16 * k + n] = h[k];
    }
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

template <typename T, int VEC, int NW, bool PART, int S = 1, int CONV = 0>
void launch_scan(const FwdParams &p, hipStream_t stream) {
    const int zslices = S > 1 ? 1 : state_slices(p.nstate);
    const dim3 grid(static_cast<unsigned>((p.dim + 4 * NW - 1) / (4 * NW)),
                    static_cast<unsigned>(p.batch), static_cast<unsigned>(zslices * p.nseg));
    hipLaunchKernelGGL((ss_fwd_kernel<T, VEC, NW, PART, S, CONV>), grid, dim3(64 * NW), 0, stream, p);
}

template <typename T, int CONV = 0>
void launch_summaries(const FwdParams &p, bool vec, hipStream_t stream) {
    constexpr int kVec = 16 / sizeof(T);
    const dim3 grid(static_cast<unsigned>((p.dim + 15) / 16), static_cast<unsigned>(p.batch),
                    static_cast<unsigned>(state_slices(p.nstate) * (p.nseg - 1)));
    if (vec) hipLaunchKernelGGL((ss_fwd_summary_kernel<T, kVec, CONV>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((ss_fwd_summary_kernel<T, 1, CONV>), grid, dim3(256), 0, stream, p);
}

template <typename T, bool PART, int S = 1, int CONV = 0>
void launch_scan_vec(const FwdParams &p, bool vec, hipStream_t stream) {
    constexpr int kVec = 16 / sizeof(T);
    if (p.nseg > 1) launch_summaries<T, CONV>(p, vec, stream);   // the segments' summaries first
    if (vec) launch_scan<T, kVec, 4, PART, S, CONV>(p, stream);
    else launch_scan<T, 1, 4, PART, S, CONV>(p, stream);
}

// up to kMaxLaneSlices slices, all in the lane
template <typename T, int CONV>
void launch_lane_slices(const FwdParams &p, bool vec, hipStream_t stream) {
    switch (state_slices(p.nstate)) {
        case 1: launch_scan_vec<T, false, 1, CONV>(p, vec, stream); break;
        case 2: launch_scan_vec<T, false, 2, CONV>(p, vec, stream); break;
        case 3: launch_scan_vec<T, false, 3, CONV>(p, vec, stream); break;
        default: launch_scan_vec<T, false, 4, CONV>(p, vec, stream); break;
    }
}

// part of the forward workspace taken by per-slice partial outputs (floats)
size_t partial_floats(int64_t batch, int64_t dim, int64_t seqlen, int nstate) {
    const int slices = state_slices(nstate);
    return slices > kMaxLaneSlices ? size_t(slices) * batch * dim * seqlen : 0;
}

template <typename T>
hipError_t launch_typed(const FwdParams &p0, hipStream_t stream) {
    // 16-byte vectors need every row start aligned: seqlen * sizeof(T) % 16 == 0
    // 4 wavefronts per workgroup: 12 would cut the B / C reads by two thirds,
    // but this pass is not bound by memory, and independent workgroups per
    // compute unit overlap their barriers.
    FwdParams p = p0;
    const bool vec = (p.seqlen * static_cast<int64_t>(sizeof(T))) % 16 == 0;
    const int slices = state_slices(p.nstate);
    p.nseg = scan_segments(p.dim, p.nstate, p.seqlen, &p.seg_len);
    if (p.nseg > 1) {   // summaries after the slice partials in the workspace
        const size_t part = partial_floats(p.batch, p.dim, p.seqlen, p.nstate);
        p.summ = static_cast<float *>(p.ypart) + (part + 63) / 64 * 64;
    }
    if (slices <= kMaxLaneSlices) {
        // the fused convolution: width 4 (the Mamba block's) fixed at compile
        // time, other widths read at run time
        if (p.conv_width == 4) launch_lane_slices<T, 4>(p, vec, stream);
        else if (p.conv_width > 0) launch_lane_slices<T, -1>(p, vec, stream);
        else launch_lane_slices<T, 0>(p, vec, stream);
        profile_mark(stream);
        return hipGetLastError();
    }
    if (p.conv_width > 0) return hipErrorInvalidValue;   // the ABI admits it up to 64 states
    // the slices see no D term and no gate; the combine adds them
    FwdParams q = p;
    q.D = nullptr;
    q.z = nullptr;
    q.ypre = nullptr;
    launch_scan_vec<T, true>(q, vec, stream);
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
    if (batch <= 0 || dim <= 0 || seqlen <= 0) return 0;
    const int slices = state_slices(nstate);
    int seg_len = 0;
    const int nseg = scan_segments(dim, nstate, seqlen, &seg_len);
    const size_t part = partial_floats(batch, dim, seqlen, nstate);
    const size_t summ = nseg > 1 ? 2 * size_t(slices) * (nseg - 1) * batch * dim * kN : 0;
    if (part + summ == 0) return 0;
    return ((part + 63) / 64 * 64 + summ) * sizeof(float);
}

hipError_t launch_fwd_summaries(const FwdParams &p, bool bf16, hipStream_t stream) {
    if (p.batch == 0 || p.dim == 0 || p.nseg < 2) return hipSuccess;
    const bool vec = (p.seqlen * (bf16 ? 2 : 4)) % 16 == 0;
    if (p.conv_width == 4) {
        if (bf16) launch_summaries<bf16_t, 4>(p, vec, stream);
        else launch_summaries<float, 4>(p, vec, stream);
    } else if (p.conv_width > 0) {
        if (bf16) launch_summaries<bf16_t, -1>(p, vec, stream);
        else launch_summaries<float, -1>(p, vec, stream);
    } else {
        if (bf16) launch_summaries<bf16_t>(p, vec, stream);
        else launch_summaries<float>(p, vec, stream);
    }
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams &p, bool bf16, hipStream_t stream) {
    if (p.batch == 0 || p.dim == 0) return hipSuccess;
    return bf16 ? launch_typed<bf16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssk
