// ss_bwd.hip -- reverse-time (BPTT) backward of the selective scan, gfx950.
//
// The loss is L = sum(dout * y) + sum(dlast * last_state).  With
// dy_t = dout_t silu(z_t) the gradient at the pre-gate output, the adjoint
// of the state obeys, backward in time,
//   g_t[n] = C[n,t] dy_t + exp(delta_{t+1} A[n]) g_{t+1}[n],   g seeded by dlast,
// and every input gradient is a sum of per-step terms:
//   du_t     = delta_t sum_n g_t B_t + D dy_t
//   ddelta_t = sum_n A_n g_t abar_t h_{t-1} + u_t sum_n g_t B_t    (times
//              sigmoid(raw + bias) when softplus is applied)
//   dz_t     = dout_t ypre_t sigmoid(z)(1 + z(1 - sigmoid(z)))
//   dB[n,t]  = sum_d g_t delta_t u_t          dC[n,t] = sum_d dy_t h_t
//   dA[d,n]  = sum_{b,t} g_t delta_t abar_t h_{t-1}
//   dD[d]    = sum_{b,t} dy_t u_t               dbias[d] = sum_{b,t} ddelta_t
// (the full backward pass through the recurrent state of the mamba-rs README,
// "Features").
//
// Three kernels on the caller's stream:
//   1. checkpoint (only when the forward did not save them): the forward
//      recurrence again, writing the state entering every 16-step block to
//      the workspace;
//   2. reverse: one lane per (channel, state) as in the forward, workgroups
//      of 16 or 48 channels (4 or 12 wavefronts).  32-step chunks are
//      visited last to first; each 16-step block re-runs its forward steps
//      from its checkpoint, keeping every decay and state in registers, then
//      walks the steps backward.
//        - sums over the 16 states (the two sums behind du and ddelta) are a
//          register butterfly of DPP adds (the first two levels select by
//          bank mask, the last two with a select);
//        - sums over channels (dB, dC): the 4 rows of a wavefront are added
//          in registers with the gfx950 cross-row lane swaps
//          (v_permlane32_swap, then v_permlane16_swap), two quantities at two
//          steps per pair of swaps, so each lane ends with one finished
//          4-row sum; the wavefronts' sums go through LDS (two buffers) and
//          are added up during the next chunk into one partial per group.
//          (f32 MFMAs could do the 4-row contraction too, but they do not
//          overlap with VALU work on this chip and would use 1/16 of each
//          instruction here);
//        - B and C are staged through two LDS buffers; u, delta, z and dout
//          are loaded by the lane that owns each element, a chunk ahead;
//   3. fold: adds the dB/dC partials over channel groups in ascending group
//      order and the dA/dD/dbias partials over the batch (and time segments)
//      in ascending order.
// A long sequence over few channels is cut into the forward's time
// segments (scan_segments, from dim, dstate and seqlen only), each run by
// its own workgroups: the block states segment by segment after the
// forward's summary pass, and the reverse pass segment by segment after an
// adjoint summary pass -- each segment but the first, from a zero adjoint,
// records the adjoint leaving its first step and the segment's total decay,
// and a segment's entering adjoint combines those of the segments after it,
// from the last down.
// Every sum runs in an order fixed by the shape, with no atomics.
#include <mutex>
#include <type_traits>

#include "ss_conv_lane.h"
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_tiles.h"

namespace ssk {
namespace {

constexpr int kRows = 16;
constexpr int kCk = kCkptSpacing;  // checkpoint spacing = reverse-pass recompute block
#ifndef SS_REV_CHUNK
#define SS_REV_CHUNK 32
#endif
constexpr int kC = SS_REV_CHUNK;   // reverse-pass staging chunk: kNB recompute blocks
constexpr int kNB = kC / kCk;
static_assert(kCk == 16 && (kNB == 1 || kNB == 2), "a staging chunk holds one or two 16-step blocks");
constexpr int kThreads = 256;

// Workspace carve-up (all f32, 256-byte aligned pieces).  With several
// 16-state slices the block states hold every slice, the partials of the
// sums over channels, batch and time come once per slice (slice k's at
// slice_bytes k further on, see slice_ws), and three (slice, batch, dim, L)
// buffers take the per-slice partial du, ddelta and dz.
struct Workspace {
    float *ckpt;     // (slice, batch, dim, nck, 16): state entering each 16-step block
    const float *ypre;  // pre-gate output saved by the forward, or nullptr
    float *dBp;      // (batch, groups, 16, L); sized for 16-channel groups
    float *dCp;      // (batch, groups, 16, L)
    int64_t groups;  // partials per (batch, state, step) that the reverse pass wrote
    int sub;         // 16-channel blocks per partial (1: 16-channel groups, 3: 48)
    float *dAp;      // (batch, dim, 16)
    float *dDp;      // (batch, dim)
    float *dbiasp;   // (batch, dim)
    size_t slice_bytes;       // distance between two slices' dBp .. dbiasp
    float *dup, *ddp, *dzp;   // several slices: (slice, batch, dim, L) partials
    int nseg;        // time segments (1: one pass over the sequence)
    int seg_len;     // steps per segment (a multiple of 64; the last takes the rest)
    float *fsumm;    // nseg > 1, block states recomputed here: the forward's segment summaries
    float *asumm;    // nseg > 1: the adjoint's segment summaries (segments 1 .. nseg - 1)
    // the fused convolution, per (batch, segment, dim): its weight-gradient
    // partials by lag (4) and bias-gradient partial; the pre-activation
    // gradients of a segment's first 4 steps and the partial input
    // gradients of its last 4 (completed across segments by a fix-up pass)
    float *dcwp, *dcbp, *dpre_head, *dx_tail;
    // 2..kMaxLaneSlices slices without the forward's record: the pre-gate
    // output the forward kernel writes for this call (batch, dim, L)
    float *ypre_ws;
    // Slices chained one launch after another (when no dz partials are
    // needed): slice slice_base of the launch; chain 0 writes the slice's
    // partial du and ddelta, 1 adds the partial to the sum of the slices
    // before it (slice 0's buffers, in place), 2 (the last slice) adds it,
    // adds the skip term with chainD and stores du and ddelta in the io
    // type.  The sums run in ascending slice order, as the combine kernel
    // adds them.
    int chain, slice_base;
    const float *chainD;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// `groups`: the dB / dC partials per batch entry the buffer holds room for;
// `with_ckpt`: whether it holds the block states (not needed when the
// forward's saved record is passed).  ss_bwd's workspace always has both at
// their largest (16-channel groups); the allocation-free entry sizes them
// for the call.  The dA / dD / dbias partials come per time segment, in
// (batch, segment, ...) order.
inline Workspace carve(void *base, int64_t batch, int64_t dim, int64_t L, int nstate,
                       int64_t groups, bool with_ckpt, size_t *total) {
    const int64_t nck = (L + kCk - 1) / kCk;
    const int slices = state_slices(nstate);
    int seg_len = 0;
    const int nseg = scan_segments(dim, nstate, L, &seg_len);
    const size_t summ = nseg > 1 ? 2 * seg_summ_half(nstate, nseg, batch, dim) : 0;
    size_t off = 0;
    Workspace w;
    char *p = static_cast<char *>(base);
    auto take = [&](size_t floats) {
        float *r = reinterpret_cast<float *>(p + off);
        off += align256(floats * sizeof(float));
        return r;
    };
    w.ckpt = with_ckpt ? take(size_t(slices) * batch * dim * nck * kN) : nullptr;
    w.ypre = nullptr;
    w.nseg = nseg;
    w.seg_len = seg_len;
    w.fsumm = (with_ckpt && summ) ? take(summ) : nullptr;
    w.asumm = summ ? take(summ) : nullptr;
    const size_t first = off;
    w.dBp = take(size_t(batch) * groups * kN * L);
    w.dCp = take(size_t(batch) * groups * kN * L);
    w.groups = groups;
    w.sub = 1;
    w.dAp = take(size_t(batch) * nseg * dim * kN);
    w.dDp = take(size_t(batch) * nseg * dim);
    w.dbiasp = take(size_t(batch) * nseg * dim);
    w.slice_bytes = off - first;
    off += (slices - 1) * w.slice_bytes;
    const size_t bsd = size_t(batch) * nseg * dim;
    w.dcwp = take(bsd * kConvMaxWidth);
    w.dcbp = take(bsd);
    w.dpre_head = take(bsd * kConvMaxWidth);
    w.dx_tail = take(bsd * kConvMaxWidth);
    w.dup = w.ddp = w.dzp = nullptr;
    w.chain = 0;
    w.slice_base = 0;
    w.chainD = nullptr;
    w.ypre_ws = nullptr;
    if (slices > 1) {
        // up to kMaxLaneSlices slices dz comes whole from the pre-gate output
        // (the caller's record, or one built here); above, from partials
        const size_t e = size_t(slices) * batch * dim * L;
        w.dup = take(e);
        w.ddp = take(e);
        if (slices > kMaxLaneSlices) w.dzp = take(e);
        else if (with_ckpt) w.ypre_ws = take(size_t(batch) * dim * L);
    }
    if (total) *total = off;
    return w;
}

// The per-slice partial pointers of slice k.
__host__ __device__ inline Workspace slice_ws(Workspace w, int k) {
    const size_t sh = size_t(k) * w.slice_bytes / sizeof(float);
    w.dBp += sh;
    w.dCp += sh;
    w.dAp += sh;
    w.dDp += sh;
    w.dbiasp += sh;
    return w;
}

// value of lane (n + 8) mod 16 of the same DPP row
__device__ __forceinline__ float row_ror8(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
}

// Sums over the 4 DPP rows of a wavefront (rows = lanes 16 k .. 16 k + 15).
// v_permlane32_swap trades lanes 32-63 of its first operand with lanes 0-31
// of its second; v_permlane16_swap trades the odd rows of its first operand
// with the even rows of its second.
//
// Sum of the two results of a lane swap.  The elements are copied out by
// value first: clang 22 takes __builtin_bit_cast of a vector element from the
// vector's first element.
template <typename V>
__device__ __forceinline__ float swap_sum(const V &r) {
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// rows_pair_sum(x, y) = [x0 + x2, x1 + x3, y0 + y2, y1 + y3]   (by row)
__device__ __forceinline__ float rows_pair_sum(float x, float y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, y), false, false);
    return swap_sum(r);
}
// rows_quad_sum(p, q) with p, q from rows_pair_sum =
//   [p0 + p1, q0 + q1, p2 + p3, q2 + q3]: row 0 holds the full 4-row sum of
//   p's x, row 1 that of q's x, rows 2 and 3 those of p's and q's y.
__device__ __forceinline__ float rows_quad_sum(float p, float q) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, p),
                                                    __builtin_bit_cast(unsigned, q), false, false);
    return swap_sum(r);
}


// ---------------------------------------------------------------------------
// kernel 1: checkpoints (64-step staging chunks, a checkpoint every 32 steps)
// ---------------------------------------------------------------------------
constexpr int kT1 = 64;
constexpr int kPitch1 = kT1 + 4;

template <typename T>
struct CkptSmem {
    static constexpr uint32_t kB = 0;
    static constexpr uint32_t kU = kB + kN * kPitch1 * 4;
    static constexpr uint32_t kDl = kU + kRows * kT1 * sizeof(T);
    static constexpr uint32_t kSize = kDl + kRows * kT1 * sizeof(T);
};

template <int J>
__device__ __forceinline__ void fwd_step(float dl, float dlu, float a2, float b, float &h) {
    h = __builtin_fmaf(exp2_hw(row_bcast<J>(dl) * a2), h, row_bcast<J>(dlu) * b);
}

// CONV: 0, or the fused convolution's width (4, or -1: read at run time);
// the u tile then holds the convolution's input
template <typename T, int VEC, int CONV = 0>
__global__ __launch_bounds__(kThreads) void ss_bwd_ckpt_kernel(BwdParams p, Workspace ws) {
    using SM = CkptSmem<T>;
    // two buffers: the next chunk is stashed into the other while this one
    // is read (one barrier per chunk)
    __shared__ __attribute__((aligned(16))) char smem[2 * SM::kSize];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, r = wave * 4 + (lane >> 4);
    const int64_t L = p.seqlen, Dm = p.dim, b = blockIdx.y;
    const int64_t d0 = int64_t(blockIdx.x) * kRows, d = d0 + r;
    const bool row_ok = d < Dm;
    const int valid_rows = int(Dm - d0 < kRows ? Dm - d0 : kRows);
    // grid z: (slice, time segment).  This slice holds states s0 .. s0 + Ns
    // - 1 of Nst; lanes n >= Ns carry zero A and B
    const int nsg = ws.nseg;
    const int slice = int(blockIdx.z) / nsg, seg = int(blockIdx.z) % nsg;
    const int Nst = p.nstate, s0 = 16 * slice;
    const int Ns = Nst - s0 < kN ? Nst - s0 : kN;
    const bool st_ok = row_ok && n < Ns;
    const float a2 = st_ok ? p.A[d * Nst + s0 + n] * kLog2e : 0.0f;
    const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    float h = (st_ok && p.h0) ? p.h0[(b * Dm + d) * Nst + s0 + n] : 0.0f;
    if (seg > 0 && row_ok) {
        // the state entering this segment, as the forward forms it: the
        // earlier segments' (decay, end state from zero) in ascending order
        const float *sh = ws.fsumm, *sd = ws.fsumm + seg_summ_half(Nst, nsg, p.batch, Dm);
        for (int j = 0; j < seg; j++) {
            const size_t i = seg_summ_index(nsg, p.batch, Dm, slice, j, b, d, n);
            h = __builtin_fmaf(sd[i], h, sh[i]);
        }
    }
    const int64_t nck = (L + kCk - 1) / kCk;
    float *ck = ws.ckpt + slice * ckpt_state_floats(p.batch, Dm, L) +
                (b * Dm + (row_ok ? d : 0)) * nck * kN + n;

    const T *gB = static_cast<const T *>(p.B) + (b * Nst + s0) * L;
    const bool zero_dead = Ns < kN;   // B rows past dstate must read as zeros
    const T *gu = static_cast<const T *>(p.u) + (b * Dm + d0) * L;
    const T *gdl = static_cast<const T *>(p.delta) + (b * Dm + d0) * L;
    ChunkStager<T, VEC, kT1, 3, kThreads> st;
    st.init(
        [&](int i) -> TileSrc<T> {
            switch (i) {
                case 0: return {gB, L, Ns, SM::kB, kPitch1, true};
                case 1: return {gu, L, valid_rows, SM::kU, kT1, false};
                default: return {gdl, L, valid_rows, SM::kDl, kT1, false};
            }
        },
        tid);

    // this segment's 64-step chunks (segments are whole chunks but the last)
    const int64_t tbeg = int64_t(seg) * ws.seg_len;
    const int64_t tend = tbeg + ws.seg_len < L ? tbeg + ws.seg_len : L;
    const int64_t cbeg = tbeg / kT1, cend = (tend + kT1 - 1) / kT1;
    ConvLane cv{};
    float xprev = 0.0f;   // the lane's convolution input one block before
    if constexpr (CONV != 0) {
        cv = conv_lane(p, d, row_ok);
        xprev = conv_prev<T>(p, b, d, row_ok, tbeg, n);
    }
    if (cend > cbeg) {
        st.fetch(cbeg * kT1, L, tid);
        st.stash(smem, zero_dead);
    }
    __syncthreads();
    for (int64_t c = cbeg; c < cend; c++) {
        const int64_t t0 = c * kT1;
        char *buf = smem + ((c - cbeg) & 1) * SM::kSize;
        float(*sB)[kPitch1] = reinterpret_cast<float(*)[kPitch1]>(buf + SM::kB);
        T(*sU)[kT1] = reinterpret_cast<T(*)[kT1]>(buf + SM::kU);
        T(*sDl)[kT1] = reinterpret_cast<T(*)[kT1]>(buf + SM::kDl);
        if (c + 1 < cend) st.fetch(t0 + kT1, L, tid);
        float dl[kT1 / 16], dlu[kT1 / 16];
#pragma unroll
        for (int s = 0; s < kT1 / 16; s++) {
            const int col = 16 * s + n;
            float x = to_f32<T>(sDl[r][col]) + bias;
            if (p.softplus) x = softplus_f32(x);
            dl[s] = (t0 + col < L) ? x : 0.0f;
            float uv = to_f32<T>(sU[r][col]);
            if constexpr (CONV != 0) {
                const float xin = uv;
                uv = row_ok ? conv_u<T, (CONV > 0 ? CONV : 0)>(cv, xin, xprev) : 0.0f;
                xprev = xin;
            }
            dlu[s] = dl[s] * uv;
        }
#pragma unroll
        for (int s = 0; s < kT1 / 16; s++) {
            if (s % (kCk / 16) == 0) {
                const int64_t k = (t0 + 16 * s) / kCk;
                if (row_ok && k < nck) ck[k * kN] = h;
            }
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&sB[n][16 * s + 4 * q]);
                switch (q) {
#define SS_FSTEP4(Q)                                            \
    case Q:                                                     \
        fwd_step<4 * Q + 0>(dl[s], dlu[s], a2, b4.x, h);        \
        fwd_step<4 * Q + 1>(dl[s], dlu[s], a2, b4.y, h);        \
        fwd_step<4 * Q + 2>(dl[s], dlu[s], a2, b4.z, h);        \
        fwd_step<4 * Q + 3>(dl[s], dlu[s], a2, b4.w, h);        \
        break;
                    SS_FSTEP4(0) SS_FSTEP4(1) SS_FSTEP4(2) SS_FSTEP4(3)
#undef SS_FSTEP4
                }
            }
        }
        // the state is complete before the barrier (left free, the
        // register-only recurrence can sink past it)
        __asm__ volatile("" : "+v"(h));
        // the other buffer's last readers (the chunk before) are behind the
        // previous barrier
        if (c + 1 < cend) st.stash(smem + ((c + 1 - cbeg) & 1) * SM::kSize, zero_dead);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// kernel 1b: adjoint summaries of the time segments
// ---------------------------------------------------------------------------
// Each segment but the first, from a zero adjoint: the reverse recurrence
// g_t = c + C_t dy_t, c <- abar_t g_t over the segment's steps, last to
// first.  The adjoint leaving the segment's first step is linear in the one
// entering its last, c_out = (product of the segment's abar) c_in + c_out(0),
// so the pairs (exp(A sum delta), c_out(0)) of the later segments give each
// segment its entering adjoint.  16 channels (4 wavefronts) per workgroup;
// C, delta, z and dout staged through LDS in 64-step chunks; grid z holds
// (slice, segment - 1).
template <typename T>
struct AdjSmem {
    static constexpr uint32_t kC = 0;
    static constexpr uint32_t kDl = kC + kN * kPitch1 * 4;
    static constexpr uint32_t kZ = kDl + kRows * kT1 * sizeof(T);
    static constexpr uint32_t kG = kZ + kRows * kT1 * sizeof(T);
    static constexpr uint32_t kSize = kG + kRows * kT1 * sizeof(T);
};

// one reverse step from the carry c entering step J of a 16-step block:
// g = c + C dy, then the carry to the step before, abar g
template <int J>
__device__ __forceinline__ void adj_step(float dl, float dy, float a2, float cv, float &c) {
    c = fmac_bcast<J>(c, dy, cv);
    c *= exp2_hw(row_bcast<J>(dl) * a2);
}

template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void ss_bwd_adjoint_summary_kernel(BwdParams p, Workspace ws) {
    using SM = AdjSmem<T>;
    // two buffers, one barrier per chunk (as in the checkpoint kernel)
    __shared__ __attribute__((aligned(16))) char smem[2 * SM::kSize];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, r = wave * 4 + (lane >> 4);
    const int64_t L = p.seqlen, Dm = p.dim, b = blockIdx.y;
    const int64_t d0 = int64_t(blockIdx.x) * kRows, d = d0 + r;
    const bool row_ok = d < Dm;
    const int valid_rows = int(Dm - d0 < kRows ? Dm - d0 : kRows);
    const int nsg = ws.nseg, nz = nsg - 1;
    const int slice = int(blockIdx.z) / nz, k = int(blockIdx.z) % nz, seg = k + 1;
    const int Nst = p.nstate, s0 = 16 * slice;
    const int Ns = Nst - s0 < kN ? Nst - s0 : kN;
    const bool st_ok = row_ok && n < Ns;
    const float a2 = st_ok ? p.A[d * Nst + s0 + n] * kLog2e : 0.0f;
    const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    const bool has_z = p.z != nullptr;
    const bool zero_dead = Ns < kN;   // C rows past dstate must read as zeros
    const T *gC = static_cast<const T *>(p.C) + (b * Nst + s0) * L;
    const int64_t rows0 = (b * Dm + d0) * L;
    const T *gdl = static_cast<const T *>(p.delta) + rows0;
    const T *gz = has_z ? static_cast<const T *>(p.z) + rows0 : nullptr;
    const T *gdo = static_cast<const T *>(p.dout) + rows0;
    ChunkStager<T, VEC, kT1, 4, kThreads> st;
    st.init(
        [&](int i) -> TileSrc<T> {
            if (i == 0) return {gC, L, Ns, SM::kC, kPitch1, true};
            if (i == 1) return {gdl, L, valid_rows, SM::kDl, kT1, false};
            if (i == 2) return {gz, L, valid_rows, SM::kZ, kT1, false};
            return {gdo, L, valid_rows, SM::kG, kT1, false};
        },
        tid);
    // the segment's 64-step chunks, last to first (only the last segment
    // has a ragged end)
    const int64_t tbeg = int64_t(seg) * ws.seg_len;
    const int64_t tend = tbeg + ws.seg_len < L ? tbeg + ws.seg_len : L;
    const int64_t cbeg = tbeg / kT1, cend = (tend + kT1 - 1) / kT1;
    float c = 0.0f, dlsum = 0.0f;
    st.fetch((cend - 1) * kT1, L, tid);
    st.stash(smem, zero_dead);
    __syncthreads();
    for (int64_t ch = cend - 1; ch >= cbeg; ch--) {
        const int64_t t0 = ch * kT1;
        char *buf = smem + ((cend - 1 - ch) & 1) * SM::kSize;
        float(*sC)[kPitch1] = reinterpret_cast<float(*)[kPitch1]>(buf + SM::kC);
        const T(*sDl)[kT1] = reinterpret_cast<const T(*)[kT1]>(buf + SM::kDl);
        const T(*sZ)[kT1] = reinterpret_cast<const T(*)[kT1]>(buf + SM::kZ);
        const T(*sG)[kT1] = reinterpret_cast<const T(*)[kT1]>(buf + SM::kG);
        if (ch > cbeg) st.fetch(t0 - kT1, L, tid);
        float dl[kT1 / 16], dy[kT1 / 16];
#pragma unroll
        for (int s = 0; s < kT1 / 16; s++) {
            const int col = 16 * s + n;
            const bool live = row_ok && t0 + col < L;
            float x = to_f32<T>(sDl[r][col]) + bias;
            if (p.softplus) x = softplus_f32(x);
            dl[s] = live ? x : 0.0f;
            float g = to_f32<T>(sG[r][col]);
            if (has_z) {
                const float zz = to_f32<T>(sZ[r][col]);
                g *= zz * sigmoid_f32(zz);
            }
            dy[s] = live ? g : 0.0f;
            dlsum += dl[s];
        }
#pragma unroll
        for (int s = kT1 / 16 - 1; s >= 0; s--) {
            const float dls = dl[s], dys = dy[s];
#pragma unroll
            for (int q = 3; q >= 0; q--) {
                const float4 c4 = *reinterpret_cast<const float4 *>(&sC[n][16 * s + 4 * q]);
                switch (q) {
#define SS_ASTEP4(Q)                                       \
    case Q:                                                \
        adj_step<4 * Q + 3>(dls, dys, a2, c4.w, c);        \
        adj_step<4 * Q + 2>(dls, dys, a2, c4.z, c);        \
        adj_step<4 * Q + 1>(dls, dys, a2, c4.y, c);        \
        adj_step<4 * Q + 0>(dls, dys, a2, c4.x, c);        \
        break;
                    SS_ASTEP4(0) SS_ASTEP4(1) SS_ASTEP4(2) SS_ASTEP4(3)
#undef SS_ASTEP4
                }
            }
        }
        // the carry is complete before the barrier (left free, the
        // register-only recurrence sinks past it into the next iteration)
        __asm__ volatile("" : "+v"(c));
        if (ch > cbeg) st.stash(smem + ((cend - ch) & 1) * SM::kSize, zero_dead);
        __syncthreads();
    }
    // the decay exp(A sum delta), the delta sum formed in one fixed tree
    // over the row's 16 lanes
    const float tot = row_sum16(dlsum);
    if (row_ok) {
        const size_t i = seg_summ_index(nsg, p.batch, Dm, slice, k, b, d, n);
        ws.asumm[i] = c;
        ws.asumm[seg_summ_half(Nst, nsg, p.batch, Dm) + i] = exp2_hw(a2 * tot);
    }
}

// ---------------------------------------------------------------------------
// kernel 2: reverse pass
// ---------------------------------------------------------------------------
constexpr int kPitch2 = kC + 4;

// NW wavefronts, 4 NW channels per workgroup.  B and C (shared by all
// channels) and, for 2-byte types, the element tiles go through LDS in two
// buffers: chunk c uses buffer c & 1 while the next chunk's tiles are
// stashed into the other.
template <typename T, int NW>
struct RevSmem {
    static constexpr int kR = 4 * NW;                                 // channels
    static constexpr uint32_t kB = 0;                                 // within a buffer
    static constexpr uint32_t kCc = kB + kN * kPitch2 * 4;
    static constexpr uint32_t kU = kCc + kN * kPitch2 * 4;          // element tiles [row kR][kC]
    static constexpr uint32_t kElem = kStageElems<T> ? kR * kC * sizeof(T) : 0;
    static constexpr uint32_t kDl = kU + kElem;
    static constexpr uint32_t kZ = kDl + kElem;
    static constexpr uint32_t kG = kZ + kElem;
    static constexpr uint32_t kBC = kG + kElem;                     // one buffer
    static constexpr uint32_t kRawEnd = 2 * kBC;
    // 4-row channel sums, two chunks' worth (a chunk's are added up during
    // the next chunk): [chunk 2][wave NW][step kC][quantity 2 x state 16 + pad].
    // At the end of a chunk thread (quantity, state, step group) adds kE
    // consecutive steps over the wavefronts: 2 steps per thread when the
    // workgroup has the threads for it, else 4.  A wavefront's threads read
    // 16 (or 8) step groups x 4 (or 8) states, and the step pitch puts them
    // in 64 distinct banks.
    static constexpr uint32_t kCh = kRawEnd;
    static constexpr int kChStep = kC == 32 ? 34 : 36;
    static constexpr int kChWave = kC * kChStep;
    static constexpr int kChBuf = NW * kChWave;   // floats of one chunk's sums
    static constexpr uint32_t kSize = kCh + 2 * kChBuf * 4;   // two chunks
    static constexpr int kE = 2 * kN * kC / 2 <= 64 * NW ? 2 : 4;
    static constexpr int kSG = kC / kE;
    static_assert(2 * kN * kSG <= 64 * NW, "one channel-sum item per thread");
};

// YP: the forward saved the pre-gate output (and z is given), so dz reads it
// instead of recomputing the sum of C h over the states.
// NW: wavefronts per workgroup (4 or 12; 4 NW channels).  Either way the
// launch bound leaves 3 wavefronts per SIMD (2 for single-element loads).
// PART: one 16-state slice of several (grid z): du, ddelta and dz are this
// slice's f32 partials (the combine kernel adds the slices and the D terms).
// CONV: 0, or the fused convolution's width (4, or -1: read at run time):
// u is recomputed from the convolution's input, and the input gradient dx,
// the weight and bias gradients (per-row partials) and the initial window's
// gradient come out instead of du.
template <typename T, int VEC, bool YP, int NW, bool PART, int CONV = 0>
__global__ __launch_bounds__(64 * NW, NW == 4 ? (VEC == 1 ? 2 : (kC == 16 ? 4 : 3)) : 1) void ss_bwd_reverse_kernel(BwdParams p, Workspace ws) {
    using SM = RevSmem<T, NW>;
    using OutT = std::conditional_t<PART, float, T>;
    static_assert(!(PART && CONV), "the fused convolution runs with one slice");
    constexpr int KC = CONV > 0 ? CONV : 0;
    // grid z: (slice, time segment)
    const int nsg = ws.nseg;
    const int slice = ws.slice_base + int(blockIdx.z) / nsg, seg = int(blockIdx.z) % nsg;
    const int chain = PART ? ws.chain : 0;
    if (PART) ws = slice_ws(ws, slice);
    constexpr bool kStage = kStageElems<T>;
    constexpr int kRowsG = SM::kR;
    constexpr int kThr = 64 * NW;
    __shared__ __attribute__((aligned(16))) char smem[SM::kSize];
    float *chan = reinterpret_cast<float *>(smem + SM::kCh);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rw = lane >> 4, n = lane & 15, r = wave * 4 + rw;
    const int64_t L = p.seqlen, Dm = p.dim, b = blockIdx.y;
    const int64_t d0 = int64_t(blockIdx.x) * kRowsG, d = d0 + r;
    const int64_t group = blockIdx.x, groups = gridDim.x;
    const bool row_ok = d < Dm;
    const int valid_rows = int(Dm - d0 < kRowsG ? Dm - d0 : kRowsG);
    const int nsub = (valid_rows + 15) / 16;   // 16-channel blocks with a valid channel
    const bool has_z = p.z != nullptr;
    // the wavefront's first row, uniform (scalar) across the wavefront
    const int64_t dw = d0 + 4 * __builtin_amdgcn_readfirstlane(wave);

    // this slice holds states s0 .. s0 + Ns - 1 of Nst; lanes n >= Ns carry
    // zero A, B, C
    const int Nst = p.nstate, s0 = 16 * slice;
    const int Ns = Nst - s0 < kN ? Nst - s0 : kN;
    const bool st_ok = row_ok && n < Ns;
    const float aval = st_ok ? p.A[d * Nst + s0 + n] : 0.0f;
    const float a2 = aval * kLog2e;
    const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    const float dskip = (row_ok && p.D) ? p.D[d] : 0.0f;
    const int64_t nck = (L + kCk - 1) / kCk;   // checkpoints (16-step blocks)
    // this segment's 32-step staging chunks cbeg .. cend - 1 (segments are
    // whole chunks but the last)
    const int64_t tbeg = int64_t(seg) * ws.seg_len;
    const int64_t tend = tbeg + ws.seg_len < L ? tbeg + ws.seg_len : L;
    const int cbeg = int(tbeg / kC), cend = int((tend + kC - 1) / kC);
    // fused convolution: this (batch, segment, row)'s partials, and the
    // first of a segment's last H steps, whose input gradients need the next
    // segment's first pre-activation gradients (none for the last segment)
    const size_t bsd = (size_t(b) * nsg + seg) * size_t(Dm) + size_t(row_ok ? d : 0);
    const int tail_start = (CONV != 0 && seg < nsg - 1) ? int(tend) - (p.conv_width - 1) : int(L);
    // Inside the chunk loop indices are 32-bit (seqlen <= 2^26), and global
    // accesses address the wavefront's 4 rows from a scalar base with 32-bit
    // byte offsets (4 rows x seqlen x 4 bytes < 2^32).
    // Lanes of rows past the last channel load the last channel's row
    // instead: in bounds, their values are not used and their stores are
    // skipped, so the loads of whole chunks need no guard.
    const int Ls = int(L), nckS = int(nck);
    const int64_t dwc = dw < Dm ? dw : Dm - 1;
    const int rwc = int((row_ok ? d : Dm - 1) - dwc);
    const float *ckb = ws.ckpt + slice * ckpt_state_floats(p.batch, Dm, L) + (b * Dm + dwc) * nck * kN;
    const uint32_t ckoff = uint32_t((rwc * nckS * kN + n) * 4);
    // state entering block k; a block past the end (only padding steps) has none
    auto ckpt_at = [&](int k) {
        return (row_ok && k >= 0 && k < nckS) ? ld_global(at_bytes(ckb, ckoff + uint32_t(k * kN * 4)))
                                              : 0.0f;
    };

    float g = (st_ok && p.dlast) ? p.dlast[(b * Dm + d) * Nst + s0 + n] : 0.0f;
    if (seg < nsg - 1 && row_ok) {
        // the adjoint entering this segment's last step: the later segments'
        // (decay, adjoint from zero) applied from the last segment down
        const float *sa = ws.asumm, *sd = ws.asumm + seg_summ_half(Nst, nsg, p.batch, Dm);
        for (int j = nsg - 1; j > seg; j--) {
            const size_t i = seg_summ_index(nsg, p.batch, Dm, slice, j - 1, b, d, n);
            g = __builtin_fmaf(sd[i], g, sa[i]);
        }
    }
    float dA_acc = 0.0f;     // this lane's state entry, summed over time
    float dD_acc = 0.0f;     // elements owned by this lane
    float dbias_acc = 0.0f;
    // fused convolution: its taps, the weight (by lag) and bias gradients of
    // the lane's elements, and the pre-activation gradients of the block
    // after the current one (zero past the segment's end)
    ConvLane cv{};
    float dwl[kConvMaxWidth] = {}, dcb = 0.0f, gnext = 0.0f;
    if constexpr (CONV != 0) cv = conv_lane(p, d, row_ok);

    const T *gB = static_cast<const T *>(p.B) + (b * Nst + s0) * L;
    const T *gC = static_cast<const T *>(p.C) + (b * Nst + s0) * L;
    const bool zero_dead = Ns < kN;   // B / C rows past dstate must read as zeros
    // this lane's row of the element-wise tensors; a row's 16 lanes load and
    // store 16 consecutive elements of a 16-step block
    const int64_t wavebase = (b * Dm + dwc) * L;
    const T *gu = static_cast<const T *>(p.u) + wavebase;
    const T *gdl = static_cast<const T *>(p.delta) + wavebase;
    const T *gz = has_z ? static_cast<const T *>(p.z) + wavebase : nullptr;
    const T *gdo = static_cast<const T *>(p.dout) + wavebase;
    const size_t slice_el = (PART && chain == 0) ? slice * size_t(p.batch * Dm * L) : 0;
    OutT *du_b = (PART ? reinterpret_cast<OutT *>(ws.dup + slice_el) : static_cast<OutT *>(p.du)) + wavebase;
    OutT *dd_b = (PART ? reinterpret_cast<OutT *>(ws.ddp + slice_el) : static_cast<OutT *>(p.ddelta)) + wavebase;
    OutT *dz_b = has_z ? (PART ? reinterpret_cast<OutT *>(ws.dzp + slice_el) : static_cast<OutT *>(p.dz)) + wavebase
                       : nullptr;
    OutT *dx_b = CONV != 0 ? static_cast<OutT *>(p.dx) + wavebase : nullptr;
    // slices with the saved pre-gate output: dz is whole, written by slice 0
    T *dz_whole = (PART && YP && has_z && slice == 0) ? static_cast<T *>(p.dz) + wavebase : nullptr;
    // the last of chained slices: the outputs in the io type, and the skip term
    T *du_fin = static_cast<T *>(p.du) + wavebase;
    T *dd_fin = static_cast<T *>(p.ddelta) + wavebase;
    const float dlast = (chain == 2 && row_ok && ws.chainD) ? ws.chainD[d] : 0.0f;
    const int rowel = rwc * Ls;   // this lane's row, in elements from the wavefront's first
    auto elem_off = [&](int t) { return uint32_t(rowel + t) * uint32_t(sizeof(T)); };
    auto out_off = [&](int t) { return uint32_t(rowel + t) * uint32_t(sizeof(OutT)); };
    // the saved pre-gate output: each owner lane loads its elements straight
    // from global memory, a chunk ahead (a row's 16 lanes read 16 floats)
    const float *ypb = ws.ypre + wavebase;
    auto ypre_at = [&](int t) {
        return (YP && row_ok && t >= 0 && t < Ls) ? ld_global(at_bytes(ypb, uint32_t(rowel + t) * 4u))
                                                  : 0.0f;
    };
    // chained slices: the earlier slices' sum of a partial, loaded the same way
    auto acc_at = [&](const OutT *base, int t) {
        return (row_ok && t >= 0 && t < Ls) ? float(ld_global(at_bytes(base, out_off(t)))) : 0.0f;
    };
    // element t of this lane's row of u, delta, z or dout (0 past the end
    // and for rows past the last channel)
    auto elem_at = [&](const T *g, int t) {
        return (row_ok && t < Ls) ? to_f32<T>(ld_global(at_bytes(g, elem_off(t)))) : 0.0f;
    };
    // B and C tiles of a chunk (and the element tiles of the group's rows
    // when staged) through LDS
    const int64_t groupbase = (b * Dm + d0) * L;
    constexpr int kPieces = kRowsG / 16;
    ChunkStager<T, VEC, kC, kStage ? 2 + 4 * kPieces : 2, kThr> st;
    st.init(
        [&](int i) -> TileSrc<T> {
            if (i == 0) return {gB, L, Ns, SM::kB, kPitch2, true};
            if (i == 1) return {gC, L, Ns, SM::kCc, kPitch2, true};
            // element tiles in 16-row pieces; a piece with no valid row points
            // at the group's first row (it is not read)
            const int q = (i - 2) / kPieces, j = (i - 2) % kPieces;
            const void *src = q == 0 ? p.u : q == 1 ? p.delta : q == 2 ? p.z : p.dout;
            const T *g = src ? static_cast<const T *>(src) + groupbase : nullptr;
            const uint32_t lds = q == 0 ? SM::kU : q == 1 ? SM::kDl : q == 2 ? SM::kZ : SM::kG;
            const int vr = valid_rows - 16 * j;
            return {(g && vr > 0) ? g + int64_t(16 * j) * L : g, L, vr > 16 ? 16 : (vr > 0 ? vr : 0),
                    lds + uint32_t(16 * j * kC * sizeof(T)), kC, false};
        },
        tid);


    // this lane's slot of the channel sums: lane (rw, n) receives state n of
    // quantity rw / 2 (0: dB, 1: dC) at the odd (rw & 1) step of a pair
    float *chw0 = chan + wave * SM::kChWave + (rw & 1) * SM::kChStep + (rw >> 1) * kN + n;
    // Adds up the wavefronts' channel sums of the chunk at tc (buffer cb):
    // thread (quantity cq, state cn, steps kE ct .. kE ct + kE - 1),
    // wavefronts in ascending order, and stores the group's partial.
    auto chan_sums = [&](int tc, int cb) {
        if (tid < 2 * kN * SM::kSG) {
            constexpr int kE = SM::kE, kSG = SM::kSG;
            const int cq = __builtin_amdgcn_readfirstlane(tid / (kN * kSG));   // uniform per wavefront
            const int cn = (tid / kSG) % kN, ct = tid % kSG;
            // 16-channel blocks (4 wavefronts each, in ascending order), then
            // the blocks with a valid channel in ascending order: the order the
            // fold uses for 16-channel partials, so the bits do not depend on
            // the group size
            float acc[kE];
#pragma unroll
            for (int e = 0; e < kE; e++) {
                const float *cs = chan + cb * SM::kChBuf + (kE * ct + e) * SM::kChStep + cq * kN + cn;
                float a = cs[0];
#pragma unroll
                for (int w = 1; w < 4; w++) a += cs[w * SM::kChWave];
#pragma unroll
                for (int sbk = 1; sbk < NW / 4; sbk++) {
                    if (sbk < nsub) {
                        float t = cs[4 * sbk * SM::kChWave];
#pragma unroll
                        for (int w = 1; w < 4; w++) t += cs[(4 * sbk + w) * SM::kChWave];
                        a += t;
                    }
                }
                acc[e] = a;
            }
            float *dst = at_bytes((cq ? ws.dCp : ws.dBp) + (b * groups + group) * kN * L,
                                  uint32_t(cn * Ls + tc + kE * ct) * 4u);
            if ((Ls % kE) == 0 && tc + kE * ct + kE <= Ls) {
                if constexpr (kE == 4)
                    *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
                else
                    *reinterpret_cast<float2 *>(dst) = make_float2(acc[0], acc[1]);
            } else {
#pragma unroll
                for (int e = 0; e < kE; e++)
                    if (tc + kE * ct + e < Ls) dst[e] = acc[e];
            }
        }
    };

    // The per-lane values of a chunk (checkpoints, the saved pre-gate
    // output, the owned elements of u, delta, z, dout) are loaded during the
    // chunk before it, once that chunk's per-element phase has consumed its
    // own, so the loads land in the same registers without copies.
    // (with seqlen 0 there is no chunk and nothing is loaded)
    float hn[kNB] = {}, ypn[kNB] = {}, un[kNB] = {}, dn[kNB] = {}, zn[kNB] = {}, gn[kNB] = {};
    float aun[kNB] = {}, adn[kNB] = {};   // chained slices: the sums so far
    // fused convolution: the lane's input one block before the chunk, as raw
    // bits loaded a chunk ahead (the initial window's value for the chunk
    // at step 0)
    ConvBits<T> xhn = 0;
    const float xwin = CONV != 0 ? conv_window(p, b, d, row_ok, n) : 0.0f;
    // whole: every step of the chunk is before the segment's end (true for
    // every chunk but a segment's last), so only the row needs care, and the
    // clamped row above takes it: the loads go unguarded.
    auto load_next = [&](int tc, bool whole) {
        if constexpr (CONV != 0) xhn = conv_prev_bits<T>(p, b, d, row_ok, tc, n);
#pragma unroll
        for (int s = 0; s < kNB; s++) {
            const int t = tc + 16 * s + n;
            const int k = kNB * (tc / kC) + s;
            hn[s] = whole ? ld_global(at_bytes(ckb, ckoff + uint32_t(k * kN * 4))) : ckpt_at(k);
            if (YP) ypn[s] = whole ? ld_global(at_bytes(ypb, uint32_t(rowel + t) * 4u)) : ypre_at(t);
            if constexpr (PART) {
                if (chain) {
                    aun[s] = whole ? float(ld_global(at_bytes(du_b, out_off(t)))) : acc_at(du_b, t);
                    adn[s] = whole ? float(ld_global(at_bytes(dd_b, out_off(t)))) : acc_at(dd_b, t);
                }
            }
            if constexpr (!kStage) {
                un[s] = whole ? to_f32<T>(ld_global(at_bytes(gu, elem_off(t)))) : elem_at(gu, t);
                dn[s] = whole ? to_f32<T>(ld_global(at_bytes(gdl, elem_off(t)))) : elem_at(gdl, t);
                if (has_z) zn[s] = whole ? to_f32<T>(ld_global(at_bytes(gz, elem_off(t)))) : elem_at(gz, t);
                gn[s] = whole ? to_f32<T>(ld_global(at_bytes(gdo, elem_off(t)))) : elem_at(gdo, t);
            }
        }
    };
    // du and ddelta of one step (of the lane's row), from its owner lane;
    // with the fused convolution du is not an output
    auto store_out = [&](int t, float duv, float ddv) {
        if (row_ok && t < Ls) {
            if (PART && chain == 2) {
                st_global(at_bytes(du_fin, elem_off(t)), from_f32<T>(duv));
                st_global(at_bytes(dd_fin, elem_off(t)), from_f32<T>(ddv));
            } else {
                if constexpr (CONV == 0) st_global(at_bytes(du_b, out_off(t)), from_f32<OutT>(duv));
                st_global(at_bytes(dd_b, out_off(t)), from_f32<OutT>(ddv));
            }
        }
    };
    if (cend > cbeg) {
        load_next((cend - 1) * kC, false);
        st.fetch(int64_t(cend - 1) * kC, L, tid);
        st.stash(smem + ((cend - 1) & 1) * SM::kBC, zero_dead);
    }
    __syncthreads();

    for (int c = cend - 1; c >= cbeg; c--) {
        const int t0 = c * kC;
        float *chw = chw0 + (c & 1) * SM::kChBuf;   // this chunk's channel-sum buffer
        char *bc = smem + (c & 1) * SM::kBC;          // and its staged tiles
        float(*sB)[kPitch2] = reinterpret_cast<float(*)[kPitch2]>(bc + SM::kB);
        float(*sC)[kPitch2] = reinterpret_cast<float(*)[kPitch2]>(bc + SM::kCc);
        const T(*sU)[kC] = reinterpret_cast<const T(*)[kC]>(bc + SM::kU);
        const T(*sDl)[kC] = reinterpret_cast<const T(*)[kC]>(bc + SM::kDl);
        const T(*sZ)[kC] = reinterpret_cast<const T(*)[kC]>(bc + SM::kZ);
        const T(*sG)[kC] = reinterpret_cast<const T(*)[kC]>(bc + SM::kG);
        if constexpr (kStage) {
            // all reads before any use (a read behind a branch would wait for
            // each one in turn); z's tile is read even without z
            T su[kNB], sd[kNB], sz[kNB], sg[kNB];
#pragma unroll
            for (int s = 0; s < kNB; s++) {
                const int col = 16 * s + n;
                su[s] = sU[r][col];
                sd[s] = sDl[r][col];
                sz[s] = sZ[r][col];
                sg[s] = sG[r][col];
            }
#pragma unroll
            for (int s = 0; s < kNB; s++) {
                un[s] = to_f32<T>(su[s]);
                dn[s] = to_f32<T>(sd[s]);
                zn[s] = has_z ? to_f32<T>(sz[s]) : 0.0f;
                gn[s] = to_f32<T>(sg[s]);
            }
        }
        float hb[kNB];   // block states, used by the blocks after the reload
#pragma unroll
        for (int s = 0; s < kNB; s++) hb[s] = row_ok ? hn[s] : 0.0f;
        if (c > cbeg) st.fetch(t0 - kC, L, tid);

        // per-element values: lane (r, n) owns elements 16 s + n of its row
        float dl[kNB], dlu[kNB], uu[kNB], sgd[kNB], dout[kNB], zz[kNB], dyv[kNB];
        float acu[kNB], acd[kNB];
#pragma unroll
        for (int s = 0; s < kNB; s++) {
            acu[s] = aun[s];
            acd[s] = adn[s];
        }
        // fused convolution: the inputs by lag and d act / d pre of the
        // lane's elements (un holds the convolution's input)
        float xl[kNB][kConvMaxWidth], gpre[kNB];
        if constexpr (CONV != 0) {
            float xprv = t0 > 0 ? conv_bits_f32<T>(xhn) : xwin;
#pragma unroll
            for (int s = 0; s < kNB; s++) {
                const float xin = un[s];
                const float pre = conv_pre<KC>(cv, xin, xprv, xl[s]);
                un[s] = row_ok ? conv_act<T>(cv, pre) : 0.0f;
                gpre[s] = conv_act_grad(cv, pre);
                xprv = xin;
            }
        }
#pragma unroll
        for (int s = 0; s < kNB; s++) {
            const int col = 16 * s + n;
            const float raw = dn[s] + bias;
            float x = raw;
            sgd[s] = 1.0f;
            if (p.softplus) {
                x = softplus_f32(raw);
                sgd[s] = sigmoid_f32(raw);
            }
            // padding steps: no decay, no input.  Rows past the last channel
            // get zero delta, delta*u and dy, which keeps their g and h at
            // zero, so they add nothing to the channel sums.
            dl[s] = (row_ok && t0 + col < Ls) ? x : 0.0f;
            uu[s] = un[s];
            dlu[s] = row_ok ? dl[s] * uu[s] : 0.0f;
            dout[s] = gn[s];
            zz[s] = zn[s];
            // gradient reaching the pre-gate output; with the saved pre-gate
            // output dz is per-element too and is written here, which keeps
            // the block's recompute free of branches
            dyv[s] = dout[s];
            if (has_z) {
                const float sz = sigmoid_f32(zz[s]);
                dyv[s] = dout[s] * zz[s] * sz;
                if (YP && row_ok && t0 + col < Ls) {
                    const float dzv = dout[s] * ypn[s] * sz * (1.0f + zz[s] * (1.0f - sz));
                    if constexpr (PART) {
                        if (dz_whole) st_global(at_bytes(dz_whole, elem_off(t0 + col)), from_f32<T>(dzv));
                    } else {
                        st_global(at_bytes(dz_b, out_off(t0 + col)), from_f32<OutT>(dzv));
                    }
                }
            }
            if (!row_ok) dyv[s] = 0.0f;
        }
        if (c > cbeg) load_next(t0 - kC, true);

        // blocks last to first: recompute the block's 16 forward steps from
        // its checkpoint (decays and states in registers), then walk them back
#pragma unroll
        for (int s = kNB - 1; s >= 0; s--) {
            // the previous (later) chunk's channel sums, complete since the
            // last barrier and not rewritten before the next one; between
            // the blocks, where their reads and adds overlap the other
            // wavefronts' walks (at the chunk's start every wavefront would
            // wait on them at once)
            if (s == 0 && c < cend - 1) chan_sums(t0 + kC, (c + 1) & 1);
            const int col = 16 * s + n;
            const float hstart = hb[s];
            float ab[kCk], hs[kCk], v[kCk];
            float h = hstart;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&sB[n][16 * s + 4 * q]);
                float4 c4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (!YP) c4 = *reinterpret_cast<const float4 *>(&sC[n][16 * s + 4 * q]);
                const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
                const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int j = 4 * q + e;
                    float dj, duj;
                    switch (j) {
#define SS_BC(J) case J: dj = row_bcast<J>(dl[s]); duj = row_bcast<J>(dlu[s]); break;
                        SS_BC(0) SS_BC(1) SS_BC(2) SS_BC(3) SS_BC(4) SS_BC(5) SS_BC(6) SS_BC(7)
                        SS_BC(8) SS_BC(9) SS_BC(10) SS_BC(11) SS_BC(12) SS_BC(13) SS_BC(14)
                        default: dj = row_bcast<15>(dl[s]); duj = row_bcast<15>(dlu[s]); break;
#undef SS_BC
                    }
                    ab[j] = exp2_hw(dj * a2);
                    h = __builtin_fmaf(ab[j], h, duj * bb[e]);
                    hs[j] = h;
                    if (!YP) v[j] = cc[e] * h;
                }
            }
            const float dy = dyv[s];
            if (!YP && has_z) {
                // pre-gate output: sum of C h over the states (lane n ends
                // with its own step) plus the skip term
                const float ypre = row_transpose_sum(reinterpret_cast<const float(&)[8]>(v[0]),
                                                     reinterpret_cast<const float(&)[8]>(v[8]), n) +
                                   dskip * uu[s];
                const float sz = sigmoid_f32(zz[s]);
                if (row_ok && t0 + col < Ls)
                    st_global(at_bytes(dz_b, out_off(t0 + col)),
                              from_f32<OutT>(dout[s] * ypre * sz * (1.0f + zz[s] * (1.0f - sz))));
            }
            if (t0 + col < Ls) dD_acc = __builtin_fmaf(dy, uu[s], dD_acc);

            // ---- backward over the block, 8 steps at a time ----
            // The walk broadcasts delta and delta*u again instead of reusing
            // the recompute's broadcasts (which would keep 32 values live
            // across it and cost the recompute its folded DPP multiplies):
            // an empty asm makes its copies distinct values to the compiler.
            float dlw = dl[s], dluw = dlu[s];
            __asm__("" : "+v"(dlw), "+v"(dluw));
            float sumA = 0.0f, sumB = 0.0f;
#pragma unroll
            for (int hh = 1; hh >= 0; hh--) {
                float qa[8], qb[8];
                float xo = 0.0f, yo = 0.0f;  // dB / dC terms of the odd step of a pair
#pragma unroll
                for (int jj = 7; jj >= 0; jj--) {
                    const int j = 8 * hh + jj;
                    const int t = 16 * s + j;
                    const float hprev = j > 0 ? hs[j - 1] : hstart;
                    float gc, gp, xv, yv;
                    // g_t = C_t dy_t + abar_{t+1} g_{t+1}; gc = abar_t g_t is
                    // carried to t - 1 and gp = g_t abar_t h_{t-1}; xv and yv
                    // are this lane's terms of the channel sums dB and dC
                    switch (j) {
#define SS_BC(J)                                          \
    case J:                                               \
        g = fmac_bcast<J, J == 15>(g, dy, sC[n][t]);      \
        gc = ab[j] * g;                                   \
        gp = gc * hprev;                                  \
        dA_acc = fmac_bcast<J, J == 15>(dA_acc, dlw, gp); \
        xv = g * row_bcast<J>(dluw);                      \
        yv = hs[j] * row_bcast<J>(dy);                    \
        break;
                        SS_BC(0) SS_BC(1) SS_BC(2) SS_BC(3) SS_BC(4) SS_BC(5) SS_BC(6) SS_BC(7)
                        SS_BC(8) SS_BC(9) SS_BC(10) SS_BC(11) SS_BC(12) SS_BC(13) SS_BC(14)
                        SS_BC(15)
#undef SS_BC
                    }
                    qa[jj] = aval * gp;
                    qb[jj] = g * sB[n][t];
                    if (jj & 1) {
                        xo = xv;
                        yo = yv;
                    } else {
                        const float pe = rows_pair_sum(xv, yv);
                        const float po = rows_pair_sum(xo, yo);
                        chw[t * SM::kChStep] = rows_quad_sum(pe, po);
                    }
                    g = gc;
                }
                // sums over the 16 states: lane n < 8 gets A*g*abar*h of step
                // 8 hh + n, lane n >= 8 g*B of step 8 hh + n - 8
                const float sum = row_transpose_sum(qa, qb, n);
                const float other = row_ror8(sum);
                // owner lanes of steps 8 hh .. 8 hh + 7 pick up both sums
                if (hh == 0 && n < 8) { sumA = sum; sumB = other; }
                if (hh == 1 && n >= 8) { sumA = other; sumB = sum; }
            }
            float du = __builtin_fmaf(dl[s], sumB, dskip * dy);
            const float dd_own = __builtin_fmaf(uu[s], sumB, sumA) * sgd[s];   // this slice's
            float dd = dd_own;
            if constexpr (PART) {
                if (chain) {
                    du = acu[s] + du;
                    dd = acd[s] + dd_own;
                }
            }
            const float duo = (PART && chain == 2) ? __builtin_fmaf(dlast, dy, du) : du;
            store_out(t0 + col, duo, dd);
            if constexpr (CONV != 0) {
                // the convolution's backward: pre-activation gradient, its
                // share of the weight and bias gradients, and the input
                // gradient dx_t = sum_j wl[j] g_{t+j} (leads from the next block)
                const float g = (row_ok && t0 + col < Ls) ? du * gpre[s] : 0.0f;
#pragma unroll
                for (int j = 0; j < kConvMaxWidth; j++) dwl[j] = __builtin_fmaf(g, xl[s][j], dwl[j]);
                dcb += g;
                const float dxv = conv_dx<KC>(cv, g, gnext);
                gnext = g;
                const int t = t0 + col;
                if (row_ok && t < Ls) {
                    if (t >= tail_start)   // completed across the segment boundary later
                        ws.dx_tail[bsd * kConvMaxWidth + (t - tail_start)] = dxv;
                    else
                        st_global(at_bytes(dx_b, out_off(t)), from_f32<OutT>(dxv));
                }
            }
            // the sum takes the rounded per-element gradient (kept out of an
            // FMA with its product), whichever way the block's code is laid out
            float ddr = dd_own;
            __asm__("" : "+v"(ddr));
            if (t0 + col < Ls) dbias_acc += ddr;
        }

        // The next chunk's B / C go to the other buffer, whose last readers
        // (the chunk before this one) are behind the previous barrier.
        if (c > cbeg) st.stash(smem + ((c - 1) & 1) * SM::kBC, zero_dead);
        __syncthreads();
    }

    // the segment's first chunk, complete since the loop's last barrier
    if (cend > cbeg) chan_sums(cbeg * kC, cbeg & 1);

    // per-row partials of the parameter gradients, per (batch entry, segment)
    const int64_t bs = b * nsg + seg;
    if (row_ok) ws.dAp[(bs * Dm + d) * kN + n] = dA_acc;
    dD_acc = row_sum16(dD_acc);
    dbias_acc = row_sum16(dbias_acc);
    if (row_ok && n == 0) {
        ws.dDp[bs * Dm + d] = dD_acc;
        ws.dbiasp[bs * Dm + d] = dbias_acc;
    }
    if (p.dh0 && st_ok && seg == 0) p.dh0[(b * Dm + d) * Nst + s0 + n] = g;

    if constexpr (CONV != 0) {
        const int H = p.conv_width - 1;
        // gnext: the pre-activation gradients of the segment's first block
        if (row_ok && nsg > 1 && n < H) ws.dpre_head[bsd * kConvMaxWidth + n] = gnext;
        if (seg == 0 && p.dconv_init && H > 0) {
            // the initial window: the input gradients of a block before step 0
            const float dv = conv_dx<KC>(cv, 0.0f, gnext);
            if (row_ok && n >= 16 - H) p.dconv_init[(b * Dm + d) * H + (n - (16 - H))] = dv;
        }
        float wsum[kConvMaxWidth];
#pragma unroll
        for (int j = 0; j < kConvMaxWidth; j++) wsum[j] = row_sum16(dwl[j]);
        const float bsum = row_sum16(dcb);
        if (row_ok && n == 0) {
#pragma unroll
            for (int j = 0; j < kConvMaxWidth; j++) ws.dcwp[bsd * kConvMaxWidth + j] = wsum[j];
            ws.dcbp[bsd] = bsum;
        }
    }
}

// The fused convolution across time segments: the input gradients of a
// segment's last H steps, completed with the next segment's first
// pre-activation gradients (the remaining leads, ascending, after the ones
// inside the segment -- the order one pass would take).  Thread per
// (batch, segment < nseg - 1, row, m < H).
template <typename T>
__global__ __launch_bounds__(256) void ss_bwd_conv_fixup_kernel(BwdParams p, Workspace ws) {
    const int K = p.conv_width, H = K - 1, nsg = ws.nseg;
    const int64_t Dm = p.dim;
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= p.batch * int64_t(nsg - 1) * Dm * H) return;
    const int m = int(i % H);
    const int64_t d = (i / H) % Dm;
    const int64_t bs = i / (int64_t(H) * Dm);
    const int64_t b = bs / (nsg - 1);
    const int seg = int(bs % (nsg - 1));
    const int64_t tend = int64_t(seg + 1) * ws.seg_len;
    const size_t here = (size_t(b) * nsg + seg) * Dm + d, next = here + Dm;
    float acc = ws.dx_tail[here * kConvMaxWidth + m];
    for (int j = H - m; j < K; j++)
        acc = __builtin_fmaf(p.conv_w[d * K + (K - 1 - j)], ws.dpre_head[next * kConvMaxWidth + (m + j - H)],
                             acc);
    static_cast<T *>(p.dx)[(b * Dm + d) * p.seqlen + tend - H + m] = from_f32<T>(acc);
}

// ---------------------------------------------------------------------------
// kernel 3: fixed-order folds
// ---------------------------------------------------------------------------
// Thread i < nbc / VT folds dB and dC at VT consecutive steps; the next
// threads fold dA, then dD and dbias.  Every sum runs in ascending group
// (or batch) order; the group loop keeps 4 groups of loads in flight.
template <int VT>
__device__ __forceinline__ void fold_add(float (&acc)[VT], const float *src) {
    if constexpr (VT == 4) {
        const u32x4 r = ld_global16(src);
        // elements are converted by value (a bit cast of a vector element
        // would read element 0 under clang 22)
        acc[0] += __uint_as_float(r.x);
        acc[1] += __uint_as_float(r.y);
        acc[2] += __uint_as_float(r.z);
        acc[3] += __uint_as_float(r.w);
    } else {
        acc[0] += ld_global(src);
    }
}

template <int VT>
__device__ __forceinline__ void fold_set(float (&acc)[VT], const float *src) {
    if constexpr (VT == 4) {
        const u32x4 r = ld_global16(src);
        acc[0] = __uint_as_float(r.x);
        acc[1] = __uint_as_float(r.y);
        acc[2] = __uint_as_float(r.z);
        acc[3] = __uint_as_float(r.w);
    } else {
        acc[0] = ld_global(src);
    }
}

template <typename T, int VT>
__global__ __launch_bounds__(256) void ss_bwd_fold_kernel(BwdParams p, Workspace ws) {
    const int64_t L = p.seqlen, Dm = p.dim, Bt = p.batch;
    const int64_t groups = ws.groups;
    const int64_t Ns = p.nstate;            // all slices
    const int64_t nbc = Bt * Ns * L / VT;   // dB / dC work items (VT divides L)
    const int64_t na = Dm * Ns;             // dA elements
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < nbc) {
        // The sum over channels has one order whatever the reverse pass's
        // group size: 16-channel partials p (each summed the same way), added
        // three at a time, q = (p0 + p1) + p2, and the q in ascending order.
        // A 48-channel pass writes q itself; a 16-channel pass writes p.
        const int64_t e = i * VT;                                // (bb, n, t) element
        const int64_t bb = e / (Ns * L), rem = e - bb * Ns * L;  // rem = n * L + t
        const int64_t ns = rem / L;                              // state n: slice ns / 16
        const Workspace wk = slice_ws(ws, int(ns / kN));
        const int64_t lrem = rem - (ns - ns % kN) * L;           // n % 16 * L + t
        const int64_t stride = kN * L;                           // one partial (16 states)
        const float *pb = wk.dBp + bb * groups * stride + lrem;
        const float *pc = wk.dCp + bb * groups * stride + lrem;
        float sb[VT] = {}, sc[VT] = {};
        if (ws.sub == 1) {   // partials are the q
            int64_t gi = 0;
            for (; gi + 4 <= groups; gi += 4) {
                // the loads of 4 partials are issued before their in-order adds
#pragma unroll
                for (int k = 0; k < 4; k++) fold_add<VT>(sb, pb + (gi + k) * stride);
#pragma unroll
                for (int k = 0; k < 4; k++) fold_add<VT>(sc, pc + (gi + k) * stride);
            }
            for (; gi < groups; gi++) {
                fold_add<VT>(sb, pb + gi * stride);
                fold_add<VT>(sc, pc + gi * stride);
            }
        } else {             // partials are the p: form each q first
            for (int64_t gi = 0; gi < groups; gi += 3) {
                float qb[VT] = {}, qc[VT] = {};
                fold_set<VT>(qb, pb + gi * stride);
                fold_set<VT>(qc, pc + gi * stride);
                if (gi + 1 < groups) {
                    fold_add<VT>(qb, pb + (gi + 1) * stride);
                    fold_add<VT>(qc, pc + (gi + 1) * stride);
                }
                if (gi + 2 < groups) {
                    fold_add<VT>(qb, pb + (gi + 2) * stride);
                    fold_add<VT>(qc, pc + (gi + 2) * stride);
                }
#pragma unroll
                for (int k = 0; k < VT; k++) {
                    sb[k] += qb[k];
                    sc[k] += qc[k];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < VT; k++) {
            static_cast<T *>(p.dB)[e + k] = from_f32<T>(sb[k]);
            static_cast<T *>(p.dC)[e + k] = from_f32<T>(sc[k]);
        }
    } else if (i < nbc + na) {
        const int64_t k = i - nbc;                      // (d, n) of dA
        const int64_t nn = k % Ns;
        const float *dap = slice_ws(ws, int(nn / kN)).dAp;
        const int64_t src = (k / Ns) * kN + nn % kN;    // the 16-wide partial of n's slice
        float s = 0.0f;
        for (int64_t bs = 0; bs < Bt * ws.nseg; bs++) s += dap[bs * Dm * kN + src];
        p.dA[k] = s;
    } else if (i < nbc + na + Dm) {
        // dD from the first slice (every slice sums the same dy u); dbias
        // over (batch entry, segment), then slices, ascending
        const int64_t dd = i - nbc - na;
        const int slices = state_slices(p.nstate);
        float sD = 0.0f, sb = 0.0f;
        for (int64_t bs = 0; bs < Bt * ws.nseg; bs++) {
            sD += ws.dDp[bs * Dm + dd];
            for (int k = 0; k < slices; k++) sb += slice_ws(ws, k).dbiasp[bs * Dm + dd];
        }
        if (p.dD) p.dD[dd] = sD;
        if (p.dbias) p.dbias[dd] = sb;
    } else if (p.conv_width > 0 && i < nbc + na + Dm + Dm * p.conv_width) {
        // the fused convolution's weight gradient (d, tap k = lag K - 1 - k),
        // over (batch entry, segment) ascending
        const int K = p.conv_width;
        const int64_t k = i - nbc - na - Dm, dd = k / K, j = K - 1 - k % K;
        float s = 0.0f;
        for (int64_t bs = 0; bs < Bt * ws.nseg; bs++) s += ws.dcwp[(bs * Dm + dd) * kConvMaxWidth + j];
        p.dconv_w[k] = s;
    } else if (p.conv_width > 0 && i < nbc + na + 2 * Dm + Dm * p.conv_width) {
        const int64_t dd = i - nbc - na - Dm - Dm * p.conv_width;
        float s = 0.0f;
        for (int64_t bs = 0; bs < Bt * ws.nseg; bs++) s += ws.dcbp[bs * Dm + dd];
        if (p.dconv_b) p.dconv_b[dd] = s;
    }
}

// Several slices: du = sum of the slices' partials + D dy, ddelta = sum of
// the partials, dz = sum of the partials + dout (D u) silu'(z); the slices
// in ascending order.  Each thread takes V consecutive elements of one row
// (V = 4 when seqlen is a multiple of 4: 16-byte partial loads).
template <int V>
__device__ __forceinline__ void sum_slices(const float *src, int64_t E, int slices, float (&s)[V]) {
    if constexpr (V == 4) {
        float4 a = *reinterpret_cast<const float4 *>(src);
        for (int k = 1; k < slices; k++) {
            const float4 b = *reinterpret_cast<const float4 *>(src + k * E);
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
    } else {
        s[0] = ld_global(src);
        for (int k = 1; k < slices; k++) s[0] += ld_global(src + k * E);
    }
}

// dz_parts: dz comes from per-slice partials (else it is already whole)
template <typename T, int V>
__global__ __launch_bounds__(256) void ss_bwd_combine_kernel(BwdParams p, Workspace ws, int slices,
                                                             int dz_parts) {
    const int64_t E = p.batch * p.dim * p.seqlen;
    const int64_t e0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * V;
    if (e0 >= E) return;
    const int64_t d = (e0 / p.seqlen) % p.dim;
    const float dskip = p.D ? p.D[d] : 0.0f;
    float du[V], dd[V], dz[V];
    sum_slices<V>(ws.dup + e0, E, slices, du);
    sum_slices<V>(ws.ddp + e0, E, slices, dd);
    const bool do_dz = p.z && dz_parts;
    if (do_dz) sum_slices<V>(ws.dzp + e0, E, slices, dz);
    auto ldv = [&](const void *src, float (&v)[V]) {
        if constexpr (V == 4) ld4<T>(static_cast<const T *>(src) + e0, v);
        else v[0] = to_f32<T>(ld_global(static_cast<const T *>(src) + e0));
    };
    auto stv = [&](void *dst, const float (&v)[V]) {
        if constexpr (V == 4) st4<T>(static_cast<T *>(dst) + e0, v);
        else st_global(static_cast<T *>(dst) + e0, from_f32<T>(v[0]));
    };
    float u[V], g[V], z[V], dy[V];
    ldv(p.u, u);
    ldv(p.dout, g);
    if (p.z) ldv(p.z, z);
#pragma unroll
    for (int i = 0; i < V; i++) {
        dy[i] = g[i];
        if (p.z) {
            const float sz = sigmoid_f32(z[i]);
            dy[i] = g[i] * z[i] * sz;
            if (do_dz) dz[i] += g[i] * (dskip * u[i]) * sz * (1.0f + z[i] * (1.0f - sz));
        }
        du[i] = __builtin_fmaf(dskip, dy[i], du[i]);
    }
    if (do_dz) stv(p.dz, dz);
    stv(p.du, du);
    stv(p.ddelta, dd);
}

// Wavefronts per reverse-pass workgroup: scan_waves' choice for 16-byte
// rows and 32-step chunks, else 4.  Time segments run side by side like
// batch entries.
int reverse_waves(const BwdParams &p, bool vec) {
    if (!vec || kC != 32) return 4;
    int seg_len = 0;
    const int nseg = scan_segments(p.dim, p.nstate, p.seqlen, &seg_len);
    return scan_waves(p.batch * nseg, p.dim);
}

// zslices: the slices this launch runs side by side (grid z), from
// ws.slice_base on; 0 for all of them
template <typename T, int VEC, bool YP, int NW, bool PART = false, int CONV = 0>
void launch_reverse(const BwdParams &p, Workspace ws, hipStream_t stream, int zslices = 0) {
    const dim3 grid(unsigned((p.dim + 4 * NW - 1) / (4 * NW)), unsigned(p.batch),
                    unsigned((zslices > 0 ? zslices : state_slices(p.nstate)) * ws.nseg));
    hipLaunchKernelGGL((ss_bwd_reverse_kernel<T, VEC, YP, NW, PART, CONV>), grid, dim3(64 * NW), 0,
                       stream, p, ws);
}

// one slice with the fused convolution (CONV: its width 4, or -1)
template <typename T, int CONV>
void launch_reverse_conv(const BwdParams &p, Workspace ws, bool vec, bool yp, int nw,
                         hipStream_t stream) {
    constexpr int kVec = 16 / sizeof(T);
    if (vec && nw == 12) {
        if (yp) launch_reverse<T, kVec, true, 12, false, CONV>(p, ws, stream);
        else launch_reverse<T, kVec, false, 12, false, CONV>(p, ws, stream);
    } else if (vec) {
        if (yp) launch_reverse<T, kVec, true, 4, false, CONV>(p, ws, stream);
        else launch_reverse<T, kVec, false, 4, false, CONV>(p, ws, stream);
    } else {
        if (yp) launch_reverse<T, 1, true, 4, false, CONV>(p, ws, stream);
        else launch_reverse<T, 1, false, 4, false, CONV>(p, ws, stream);
    }
}

template <typename T, int CONV>
void launch_ckpt(const BwdParams &p, Workspace ws, bool vec, dim3 grid, hipStream_t stream) {
    constexpr int kVec = 16 / sizeof(T);
    if (vec) hipLaunchKernelGGL((ss_bwd_ckpt_kernel<T, kVec, CONV>), grid, dim3(kThreads), 0, stream, p, ws);
    else hipLaunchKernelGGL((ss_bwd_ckpt_kernel<T, 1, CONV>), grid, dim3(kThreads), 0, stream, p, ws);
}

// Channel groups of the reverse pass for this call (and so dB / dC partials
// per batch entry).
int64_t reverse_groups(const BwdParams &p, size_t esize) {
    const bool vec = (p.seqlen * int64_t(esize)) % 16 == 0;
    const int nw = reverse_waves(p, vec);
    return (p.dim + 4 * nw - 1) / (4 * nw);
}

template <typename T>
hipError_t launch_typed(const BwdParams &p, hipStream_t stream) {
    Workspace ws = p.tight_ws
                       ? carve(p.workspace, p.batch, p.dim, p.seqlen, p.nstate,
                               reverse_groups(p, sizeof(T)), p.ckpt == nullptr, nullptr)
                       : carve(p.workspace, p.batch, p.dim, p.seqlen, p.nstate,
                               (p.dim + kRows - 1) / kRows, true, nullptr);
    const int slices = state_slices(p.nstate);
    // 2..kMaxLaneSlices slices: the reverse pass takes dz whole from the
    // pre-gate output, the caller's record or one the forward kernel builds
    const bool lane_slices = slices > 1 && slices <= kMaxLaneSlices;
    if (p.ckpt) {  // saved by the forward: read only
        ws.ckpt = const_cast<float *>(p.ckpt);
        ws.ypre = slices <= kMaxLaneSlices ? p.ypre : nullptr;
    }
    if (p.batch > 0 && p.dim > 0) {
        dim3 grid(unsigned((p.dim + kRows - 1) / kRows), unsigned(p.batch), unsigned(slices * ws.nseg));
        constexpr int kVec = 16 / sizeof(T);
        const bool vec = (p.seqlen * int64_t(sizeof(T))) % 16 == 0;
        if (!p.ckpt && lane_slices) {
            // the record from the forward kernel (a row's slices in the lane):
            // block states and, with z, the pre-gate output; no out
            FwdParams fp{};
            static_cast<ScanParams &>(fp) = p;
            fp.out = nullptr;
            fp.last_state = nullptr;
            fp.ckpt = ws.ckpt;
            fp.ypre = p.z ? ws.ypre_ws : nullptr;
            fp.ypart = ws.fsumm;   // room for its time segments' summaries
            const hipError_t e = launch_fwd(fp, sizeof(T) == 2, stream);
            if (e != hipSuccess) return e;
            ws.ypre = fp.ypre;
        } else if (!p.ckpt) {
            if (ws.nseg > 1) {   // the forward's segment summaries, then the states
                FwdParams fp{};
                static_cast<ScanParams &>(fp) = p;
                fp.nseg = ws.nseg;
                fp.seg_len = ws.seg_len;
                fp.summ = ws.fsumm;
                fp.conv_width = p.conv_width;
                fp.conv_silu = p.conv_silu;
                fp.conv_w = p.conv_w;
                fp.conv_b = p.conv_b;
                fp.conv_init = p.conv_init;
                const hipError_t e = launch_fwd_summaries(fp, sizeof(T) == 2, stream);
                if (e != hipSuccess) return e;
            }
            if (p.conv_width == 4) launch_ckpt<T, 4>(p, ws, vec, grid, stream);
            else if (p.conv_width > 0) launch_ckpt<T, -1>(p, ws, vec, grid, stream);
            else launch_ckpt<T, 0>(p, ws, vec, grid, stream);
            profile_mark(stream);
        }
        if (ws.nseg > 1) {   // the adjoint's segment summaries
            const dim3 agrid(unsigned((p.dim + kRows - 1) / kRows), unsigned(p.batch),
                             unsigned(slices * (ws.nseg - 1)));
            if (vec)
                hipLaunchKernelGGL((ss_bwd_adjoint_summary_kernel<T, kVec>), agrid, dim3(kThreads), 0,
                                   stream, p, ws);
            else
                hipLaunchKernelGGL((ss_bwd_adjoint_summary_kernel<T, 1>), agrid, dim3(kThreads), 0,
                                   stream, p, ws);
            profile_mark(stream);
        }
        const bool yp = p.z && ws.ypre && (slices == 1 ? p.ckpt != nullptr : lane_slices);
        // several slices and no dz partials to add: the slices run one launch
        // after another and the last stores du and ddelta (no combine kernel)
        const bool chained = slices > 1 && (yp || !p.z) && p.conv_width == 0;
        const int nw = reverse_waves(p, vec);
        ws.groups = (p.dim + 4 * nw - 1) / (4 * nw);   // the partials the fold reads
        ws.sub = nw == 12 ? 1 : 3;
        // slices see no D term (the combine adds it and its gradients)
        BwdParams q = p;
        q.D = nullptr;
        q.ypre = nullptr;
        if (p.conv_width == 4) {
            launch_reverse_conv<T, 4>(p, ws, vec, yp, nw, stream);
        } else if (p.conv_width > 0) {
            launch_reverse_conv<T, -1>(p, ws, vec, yp, nw, stream);
        } else if (slices > 1) {
            auto part = [&](Workspace w, int zsl) {
                if (yp) {
                    if (vec && nw == 12) launch_reverse<T, kVec, true, 12, true>(q, w, stream, zsl);
                    else if (vec) launch_reverse<T, kVec, true, 4, true>(q, w, stream, zsl);
                    else launch_reverse<T, 1, true, 4, true>(q, w, stream, zsl);
                } else {
                    if (vec && nw == 12) launch_reverse<T, kVec, false, 12, true>(q, w, stream, zsl);
                    else if (vec) launch_reverse<T, kVec, false, 4, true>(q, w, stream, zsl);
                    else launch_reverse<T, 1, false, 4, true>(q, w, stream, zsl);
                }
            };
            if (chained) {   // one launch per slice, each adding to the sum so far
                for (int sl = 0; sl < slices; sl++) {
                    Workspace w = ws;
                    w.slice_base = sl;
                    w.chain = sl == 0 ? 0 : (sl == slices - 1 ? 2 : 1);
                    w.chainD = p.D;
                    part(w, 1);
                }
            } else {
                part(ws, 0);
            }
        } else if (vec && nw == 12) {
            if (yp) launch_reverse<T, kVec, true, 12>(p, ws, stream);
            else launch_reverse<T, kVec, false, 12>(p, ws, stream);
        } else if (vec) {
            if (yp) launch_reverse<T, kVec, true, 4>(p, ws, stream);
            else launch_reverse<T, kVec, false, 4>(p, ws, stream);
        } else {
            if (yp) launch_reverse<T, 1, true, 4>(p, ws, stream);
            else launch_reverse<T, 1, false, 4>(p, ws, stream);
        }
        profile_mark(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.conv_width > 1 && ws.nseg > 1) {   // the convolution across segment boundaries
            const int64_t nfix = p.batch * int64_t(ws.nseg - 1) * p.dim * (p.conv_width - 1);
            hipLaunchKernelGGL((ss_bwd_conv_fixup_kernel<T>), dim3(unsigned((nfix + 255) / 256)),
                               dim3(256), 0, stream, p, ws);
            profile_mark(stream);
        }
        const int64_t E = p.batch * p.dim * p.seqlen;
        if (slices > 1 && E > 0 && !chained) {
            if (p.seqlen % 4 == 0)
                hipLaunchKernelGGL((ss_bwd_combine_kernel<T, 4>), dim3(unsigned((E / 4 + 255) / 256)),
                                   dim3(256), 0, stream, p, ws, slices, int(!yp));
            else
                hipLaunchKernelGGL((ss_bwd_combine_kernel<T, 1>), dim3(unsigned((E + 255) / 256)),
                                   dim3(256), 0, stream, p, ws, slices, int(!yp));
            profile_mark(stream);
        }
    }
    const bool v4 = p.seqlen % 4 == 0;   // 16-byte partial loads
    const int64_t total = p.batch * p.nstate * p.seqlen / (v4 ? 4 : 1) + p.dim * p.nstate + p.dim +
                          (p.conv_width > 0 ? p.dim * (p.conv_width + 1) : 0);
    if (total == 0 && !(p.batch > 0 && p.dim > 0)) return hipSuccess;   // nothing was enqueued
    if (total > 0) {
        const dim3 fgrid(unsigned((total + 255) / 256));
        if (v4)
            hipLaunchKernelGGL((ss_bwd_fold_kernel<T, 4>), fgrid, dim3(256), 0, stream, p, ws);
        else
            hipLaunchKernelGGL((ss_bwd_fold_kernel<T, 1>), fgrid, dim3(256), 0, stream, p, ws);
        profile_mark(stream);
    }
    return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int nstate) {
    size_t total = 0;
    carve(nullptr, batch, dim, seqlen, nstate, (dim + kRows - 1) / kRows, true, &total);
    return total;
}

// ---------------------------------------------------------------------------
// Allocation-free backward: the workspace is a file-scope device array
// ---------------------------------------------------------------------------
// Every reverse pass and fold writes each workspace word it later reads
// (block states, partials), so the array needs no clearing between calls;
// it keeps the last call's contents.  Calls that overlap on one GPU share it
// and race.
static __device__ __align__(256) char scratch[kBwdScratchBytes];

size_t bwd_noalloc_bytes(const BwdParams &p, bool bf16) {
    if (p.batch <= 0 || p.dim <= 0) return 0;
    size_t total = 0;
    carve(nullptr, p.batch, p.dim, p.seqlen, p.nstate, reverse_groups(p, bf16 ? 2 : 4),
          p.ckpt == nullptr, &total);
    return total;
}

hipError_t bwd_scratch(void **ptr) {
    // each device holds its own copy of the array; its address is looked up
    // once per device, with that device current (the array's name is not a
    // device address in host code)
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_bwd(const BwdParams &p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_typed<bf16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssk
