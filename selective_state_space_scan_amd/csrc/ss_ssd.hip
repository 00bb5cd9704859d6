// ss_ssd.hip -- Mamba-2 SSD forward (scalar A per head) on gfx950 matrix cores.
//
// The state-spaces/mamba README ("Mamba-2", "SSD") names the SSD module of
// the Mamba-2 block (d_state typically 64 or 128).  Per batch b and head h,
// with a headdim x dstate state H:
//   dt_t = softplus(dt_raw[b,t,h] + dt_bias[h]),  a_t = dt_t A[h]
//   H_t  = exp(a_t) H_{t-1} + dt_t x_t B_t^T,      y_t = H_t C_t + D[h] x_t
// B and C belong to the head's group (contiguous groups of heads).
//
// Chunked form.  Time runs in chunks of kQ = 64 steps.  With cum_t the sum
// of a over the chunk up to and including t (so exp(cum_t - cum_s) is the
// decay from step s to t), a chunk's output and end state are
//   y_t   = exp(cum_t) C_t . H_in  +  sum_{s<=t} exp(cum_t - cum_s) (C_t . B_s) dt_s x_s
//   H_out = exp(cum_last) H_in    +  sum_s exp(cum_last - cum_s) dt_s x_s B_s^T
// which is the recurrence regrouped (the quadratic "dual" form inside a
// chunk, the recurrence between chunks).  All four products are dense
// contractions and run on bf16 MFMAs with f32 accumulation:
//   G^T = B C^T (over d_state; 16x16x32), Y += W X (over the chunk; 16x16x16),
//   Y += C H^T (over d_state; 16x16x16), H^T += B^T (w X) (over the chunk; 16x16x32).
//
// Work mapping.  One workgroup per (batch, head); two wavefronts own the 16
// columns 16q .. 16q + 15 of the head (see the kernel).  The state lives in
// MFMA accumulators as H^T tiles (16 states x 16 columns); their registers
// are, after the bf16 split, exactly the B operand of the C H^T product.  G^T is computed (rather than G) because its accumulator
// registers, scaled by exp(cum_t - cum_s) dt_s, are exactly the A operand of
// the W X product -- neither needs a trip through LDS.  Every wavefront
// computes the chunk's G^T itself (it is the same for all columns).
// A chunk's B, C (row-major, d_state contiguous), B^T and x^T (time
// contiguous) and dt go through LDS; the next chunk is loaded into
// registers while the current one is computed.  The chunk's output is
// gathered in LDS and written in whole 16-byte pieces of full rows (a
// head's row is headdim contiguous values): 2-byte stores of a wavefront's
// 16 columns cost more than the rest of the kernel together.
//
// Rounding: B, C, x arrive as bf16.  The three operands made on chip -- W,
// the state H and w x -- are each split into a bf16 high part and a bf16
// low part (v = hi + lo to about 2^-16 relative) and multiplied as two
// products, so they add no error beyond f32 accumulation; a single bf16
// rounding of them would cost up to 2% of the output at d_state 128, as
// each output element sums 128 state terms.  Sums and the carried state
// are f32.
#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_mfma.h"
#include "ss_tiles.h"

namespace ssk {
namespace {

constexpr int kQ = 64;  // chunk length

template <int N, int P>
struct SsdSmem {
    static constexpr int kPB = N + 8;   // row pitch of B and C (bf16), 16-byte multiple
    static constexpr int kPT = kQ + 8;  // row pitch of B^T and x^T (bf16)
    static constexpr uint32_t kBs = 0;
    static constexpr uint32_t kCs = kBs + kQ * kPB * 2;
    static constexpr uint32_t kBT = kCs + kQ * kPB * 2;
    static constexpr uint32_t kXT = kBT + N * kPT * 2;
    static constexpr uint32_t kCum = kXT + P * kPT * 2;  // f32 [kQ]
    static constexpr uint32_t kDt = kCum + kQ * 4;       // f32 [kQ]
    static constexpr uint32_t kW = kDt + kQ * 4;         // f32 [kQ]: exp(cum_last - cum_s) dt_s
    static constexpr int kPY = P + 8;                     // row pitch of the output tile (bf16)
    static constexpr uint32_t kYs = kW + kQ * 4;          // bf16 [kQ][kPY]: the chunk's output
    // state exchange, per chunk parity: [column tile][state tile][lane] x 16 bytes
    static constexpr uint32_t kHx = kYs + kQ * kPY * 2;
    static constexpr uint32_t kHxPar = (P / 16) * (N / 16) * 64 * 16;
    static constexpr uint32_t kSize = kHx + 2 * kHxPar;
};

// N: dstate (multiple of 32, <= 128); P: headdim (multiple of 16, <= 64).
// Two wavefronts per 16-column tile q: wavefront (q, hf) computes the
// outputs of time tiles {0, 3} (hf = 0) or {1, 2} (hf = 1) -- five of the
// ten lower-triangle B C^T tiles each -- and carries state tiles
// hf N / 32 .. (hf + 1) N / 32 - 1.  C H^T needs all state tiles, so after
// each chunk's update the wavefronts publish their state (as the bf16
// hi/lo operands) in an LDS exchange buffer, double-buffered by chunk.
//
// The state entering chunk c is stored to p.states, when given, as (batch,
// head, chunk) blocks of a dstate x headdim f32 matrix (headdim contiguous):
// the forward's checkpoint for the backward.  kStates: the backward's own
// states pass, when no checkpoint was saved.  Only the recurrence runs (no
// output, no C H_in, no W X), and its wavefronts need no state exchange.
template <int N, int P, bool kStates>
__global__ __launch_bounds__(8 * P) void ss_ssd_fwd_kernel(SsdParams p) {
    constexpr int kCT = P / 16;                      // column tiles
    constexpr int kWaves = 2 * kCT, kThr = 64 * kWaves;
    constexpr int kNT = N / 16, kNH = kNT / 2;       // state tiles, per wavefront
    constexpr int kVB = kQ * N / 8;                  // 16-byte vectors of a B (or C) chunk
    constexpr int kBV = (kVB + kThr - 1) / kThr;     // per thread
    constexpr int kVX = kQ * P / 8;                  // 16-byte vectors of an x chunk
    static_assert(kVX == kThr, "one x vector per thread");
    using SM = SsdSmem<N, P>;
    __shared__ __attribute__((aligned(16))) char smem[SM::kSize];
    bf16_t *Bs = reinterpret_cast<bf16_t *>(smem + SM::kBs);
    bf16_t *Cs = reinterpret_cast<bf16_t *>(smem + SM::kCs);
    bf16_t *BT = reinterpret_cast<bf16_t *>(smem + SM::kBT);
    bf16_t *XT = reinterpret_cast<bf16_t *>(smem + SM::kXT);
    float *cum = reinterpret_cast<float *>(smem + SM::kCum);
    float *dts = reinterpret_cast<float *>(smem + SM::kDt);
    float *wts = reinterpret_cast<float *>(smem + SM::kW);
    bf16_t *Ys = reinterpret_cast<bf16_t *>(smem + SM::kYs);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = wv % kCT, hf = wv / kCT;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t H = p.nheads, G = p.ngroups, L = p.seqlen;
    // consecutive workgroups go to the 8 XCDs in turn: with the batch index
    // the fast one, the heads of a batch entry (which share its B and C)
    // land on the same XCD's L2 when batch is a multiple of 8
    const int64_t b = blockIdx.x % p.batch, h = blockIdx.x / p.batch;
    const int64_t g = h / (H / G);
    const float a2 = p.A[h] * kLog2e;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const float dskip = p.D ? p.D[h] : 0.0f;
    const int64_t xrow = H * P, brow = G * N;   // element strides between time steps
    const bf16_t *xg = static_cast<const bf16_t *>(p.x) + (b * L * H + h) * P;
    const bf16_t *dtg = static_cast<const bf16_t *>(p.dt) + b * L * H + h;
    const bf16_t *Bg = static_cast<const bf16_t *>(p.B) + (b * L * G + g) * N;
    const bf16_t *Cg = static_cast<const bf16_t *>(p.C) + (b * L * G + g) * N;
    bf16_t *yg = static_cast<bf16_t *>(p.out) + (b * L * H + h) * P;

    // this wavefront's state tiles m = hf kNH + mm: lane holds
    // H^T[n = 16 m + 4 lg + r][col = 16 q + li]
    const int col = 16 * q + li;
    const int m0 = hf * kNH;
    f32x4 Hs[kNH];
    if (p.h0) {   // one test for all loads, so they are issued together
        const float *h0 = p.h0 + ((b * H + h) * P + col) * N;
#pragma unroll
        for (int mm = 0; mm < kNH; mm++)
            Hs[mm] = *reinterpret_cast<const f32x4 *>(h0 + 16 * (m0 + mm) + 4 * lg);
    } else {
#pragma unroll
        for (int mm = 0; mm < kNH; mm++) Hs[mm] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // exchange entry of state tile m of column tile q: this lane's 4 bf16
    // high parts, then its 4 low parts
    auto hx = [&](int par, int m) {
        return reinterpret_cast<s16x4 *>(smem + SM::kHx + par * SM::kHxPar +
                                         ((q * kNT + m) * 64 + lane) * 16);
    };
    auto publish = [&](int par) {
#pragma unroll
        for (int mm = 0; mm < kNH; mm++) {
            s16x4 hi, lo;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const short v = bfs(Hs[mm][r]);
                hi[r] = v;
                lo[r] = lo_bf(Hs[mm][r], v);
            }
            s16x4 *e = hx(par, m0 + mm);
            e[0] = hi;
            e[1] = lo;
        }
    };
    if constexpr (!kStates) publish(0);

    // the next chunk, in registers
    u32x4 rb[kBV], rc[kBV], rx;
    uint32_t rdt = 0;
    // Vector v of a chunk is 8 values (16 bytes) of step s = v % kQ, from
    // value 8 c8 on, c8 = v / kQ: the 64 lanes of a wavefront take 64
    // consecutive steps, so the transposed LDS writes below go to 64
    // consecutive 2-byte slots (no bank conflicts).
    auto load_chunk = [&](int64_t c0) {
#pragma unroll
        for (int k = 0; k < kBV; k++) {
            const int v = tid + k * kThr;
            if (v < kVB) {
                const int s = v % kQ, c8 = v / kQ;
                const int64_t t = c0 + s < L ? c0 + s : L - 1;
                rb[k] = ld_global16(Bg + t * brow + 8 * c8);
                if constexpr (!kStates) rc[k] = ld_global16(Cg + t * brow + 8 * c8);
            }
        }
        {
            const int s = tid % kQ, c8 = tid / kQ;
            const int64_t t = c0 + s < L ? c0 + s : L - 1;
            rx = ld_global16(xg + t * xrow + 8 * c8);
        }
        if (tid < kQ) {
            const int64_t t = c0 + tid < L ? c0 + tid : L - 1;
            rdt = ld_global(dtg + t * H);
        }
    };
    // registers -> LDS; steps past the end become zeros (no input, no decay)
    auto stash_chunk = [&](int64_t c0) {
#pragma unroll
        for (int k = 0; k < kBV; k++) {
            const int v = tid + k * kThr;
            if (v < kVB) {
                const int s = v % kQ, c8 = v / kQ;
                const bool live = c0 + s < L;
                u32x4 vb = rb[k];
                if (!live) vb = u32x4{0u, 0u, 0u, 0u};
                if constexpr (!kStates) {
                    u32x4 vc = rc[k];
                    if (!live) vc = u32x4{0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4 *>(Bs + s * SM::kPB + 8 * c8) = vb;
                    *reinterpret_cast<u32x4 *>(Cs + s * SM::kPB + 8 * c8) = vc;
                }
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    BT[(8 * c8 + 2 * e) * SM::kPT + s] = bf16_t(vb[e] & 0xffffu);
                    BT[(8 * c8 + 2 * e + 1) * SM::kPT + s] = bf16_t(vb[e] >> 16);
                }
            }
        }
        {
            const int s = tid % kQ, c8 = tid / kQ;
            u32x4 vx = rx;
            if (!(c0 + s < L)) vx = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                XT[(8 * c8 + 2 * e) * SM::kPT + s] = bf16_t(vx[e] & 0xffffu);
                XT[(8 * c8 + 2 * e + 1) * SM::kPT + s] = bf16_t(vx[e] >> 16);
            }
        }
        if (tid < kQ) {   // wavefront 0: dt, the running sum of dt A, and w
            float dv = 0.0f;
            if (c0 + tid < L) {
                dv = bf_lo(rdt & 0xffffu) + bias;
                if (p.softplus) dv = softplus_f32(dv);
            }
            // running sum of dt A in base-2 exponent units (plain f32: the
            // rounding of large sums stays far below the bf16 output's; the
            // backward, whose dA needs more, carries it compensated)
            float a = dv * a2;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(a, off, 64);
                if (lane >= off) a += o;
            }
            const float total = __shfl(a, 63, 64);
            cum[tid] = a;
            dts[tid] = dv;
            wts[tid] = exp2_hw(total - a) * dv;
        }
    };

    // One chunk for this wavefront; HF = hf as a compile-time constant so
    // that the time tiles and the triangle loops unroll.
    auto chunk = [&](auto hfc, int par) {
        constexpr int HF = decltype(hfc)::value;
        constexpr int kT[2] = {HF ? 1 : 0, HF ? 2 : 3};
        if constexpr (!kStates) {
        // C H_in, from every state tile: the 16x16x32 product runs over state
        // tiles 2 m2 and 2 m2 + 1 at once, its k index over (tile, 4 lg + r)
        // in the order the state accumulators hold them, and C is read in
        // that same order
        bf16x8_t hbh[kNT / 2], hbl[kNT / 2];
#pragma unroll
        for (int m2 = 0; m2 < kNT / 2; m2++) {
            const s16x4 *e0 = hx(par, 2 * m2), *e1 = hx(par, 2 * m2 + 1);
            const s16x4 h0v = e0[0], l0v = e0[1], h1v = e1[0], l1v = e1[1];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                // by value before the bit cast (clang 22 would read element 0)
                const short a0 = h0v[r], a1 = h1v[r], b0 = l0v[r], b1 = l1v[r];
                hbh[m2][r] = __builtin_bit_cast(__bf16, a0);
                hbh[m2][4 + r] = __builtin_bit_cast(__bf16, a1);
                hbl[m2][r] = __builtin_bit_cast(__bf16, b0);
                hbl[m2][4 + r] = __builtin_bit_cast(__bf16, b1);
            }
        }
        f32x4 Y[2];
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
            const int i = kT[ii];
            s16x4 a0[kNT / 2], a1[kNT / 2];
#pragma unroll
            for (int m2 = 0; m2 < kNT / 2; m2++) {
                const bf16_t *crow = Cs + (16 * i + li) * SM::kPB + 32 * m2 + 4 * lg;
                a0[m2] = *reinterpret_cast<const s16x4 *>(crow);
                a1[m2] = *reinterpret_cast<const s16x4 *>(crow + 16);
            }
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int m2 = 0; m2 < kNT / 2; m2++) {
                bf16x8_t a;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const short v0 = a0[m2][e], v1 = a1[m2][e];
                    a[e] = __builtin_bit_cast(__bf16, v0);
                    a[4 + e] = __builtin_bit_cast(__bf16, v1);
                }
                acc = mfma32(a, hbh[m2], acc);
                acc = mfma32(a, hbl[m2], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; r++) acc[r] *= exp2_hw(cum[16 * i + 4 * lg + r]);
            Y[ii] = acc;
        }
        // the chunk's own part: W = G . exp(cum_t - cum_s) dt_s (s <= t),
        // Y += W x.  This lane's s are 16 j + 4 lg + r and its t 16 i + li.
        f32x4 cs[4], ds[4];
        s16x4 xb[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if (j > kT[1]) break;
            cs[j] = *reinterpret_cast<const f32x4 *>(cum + 16 * j + 4 * lg);
            ds[j] = *reinterpret_cast<const f32x4 *>(dts + 16 * j + 4 * lg);
            xb[j] = *reinterpret_cast<const s16x4 *>(XT + col * SM::kPT + 16 * j + 4 * lg);
        }
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
            const int i = kT[ii];
            const int t = 16 * i + li;
            const float ct = cum[t];
            bf16x8_t cb[N / 32];
#pragma unroll
            for (int k = 0; k < N / 32; k++)
                cb[k] = *reinterpret_cast<const bf16x8_t *>(Cs + t * SM::kPB + 32 * k + 8 * lg);
#pragma unroll
            for (int j = 0; j <= i; j++) {
                bf16x8_t ba[N / 32];
#pragma unroll
                for (int k = 0; k < N / 32; k++)
                    ba[k] = *reinterpret_cast<const bf16x8_t *>(Bs + (16 * j + li) * SM::kPB + 32 * k + 8 * lg);
                f32x4 gt = {0.0f, 0.0f, 0.0f, 0.0f};   // G^T[s = 16 j + 4 lg + r][t]
#pragma unroll
                for (int k = 0; k < N / 32; k++) gt = mfma32(ba[k], cb[k], gt);
                s16x4 wh, wl;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    float wvv = gt[r] * exp2_hw(ct - cs[j][r]) * ds[j][r];
                    // below the diagonal s < t always; on it keep s <= t (a
                    // select: both sides are computed, no branch)
                    if (j == i) wvv = (4 * lg + r <= li) ? wvv : 0.0f;
                    const short hi = bfs(wvv);
                    wh[r] = hi;
                    wl[r] = lo_bf(wvv, hi);
                }
                Y[ii] = mfma16(wh, xb[j], Y[ii]);
                Y[ii] = mfma16(wl, xb[j], Y[ii]);
            }
        }
        // y + D x into the output tile (lane holds y[t = 16 i + 4 lg + r][col]);
        // it leaves in whole rows after the barrier
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int t = 16 * kT[ii] + 4 * lg + r;
                const float xv = bf16_to_f32(XT[col * SM::kPT + t]);
                Ys[t * SM::kPY + col] = f32_to_bf16(Y[ii][r] + dskip * xv);
            }
        }
        }  // !kStates
        // this wavefront's state tiles: H_out = exp(cum_last) H_in + B^T (w x)
        const float decay = exp2_hw(cum[kQ - 1]);
        bf16x8_t xsh[2], xsl[2];
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            const u32x4 xr = *reinterpret_cast<const u32x4 *>(XT + col * SM::kPT + 32 * kk + 8 * lg);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int s = 32 * kk + 8 * lg + e;
                const float v = ((e & 1) ? bf_hi(xr[e >> 1]) : bf_lo(xr[e >> 1])) * wts[s];
                const __bf16 hi = static_cast<__bf16>(v);
                xsh[kk][e] = hi;
                xsl[kk][e] = static_cast<__bf16>(v - static_cast<float>(hi));
            }
        }
#pragma unroll
        for (int mm = 0; mm < kNH; mm++) {
#pragma unroll
            for (int r = 0; r < 4; r++) Hs[mm][r] *= decay;
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(BT + (16 * (m0 + mm) + li) * SM::kPT + 32 * kk + 8 * lg);
                Hs[mm] = mfma32(a, xsh[kk], Hs[mm]);
                Hs[mm] = mfma32(a, xsl[kk], Hs[mm]);
            }
        }
    };

    const int64_t nch = (L + kQ - 1) / kQ;
    if (nch > 0) {
        load_chunk(0);
        stash_chunk(0);
    }
    __syncthreads();
    for (int64_t c = 0; c < nch; c++) {
        const int64_t c0 = c * kQ;
        if (c + 1 < nch) load_chunk(c0 + kQ);
        if (kStates || p.states) {
            // H_in of this chunk: lane holds H^T[n][col], 16 lanes one row piece
            float *st = p.states + (((b * H + h) * nch + c) * N) * P + col;
#pragma unroll
            for (int mm = 0; mm < kNH; mm++)
#pragma unroll
                for (int r = 0; r < 4; r++) st[(16 * (m0 + mm) + 4 * lg + r) * P] = Hs[mm][r];
        }
        const int par = int(c & 1);
        if (hf) chunk(std::integral_constant<int, 1>{}, par);
        else chunk(std::integral_constant<int, 0>{}, par);
        if constexpr (!kStates) {
        // the new state for the next chunk's C H_in (the other buffer: its
        // last readers were the previous chunk's, behind the last barrier)
        publish(par ^ 1);
        }
        __syncthreads();
        // the chunk's output rows: 16-byte stores, P / 8 lanes per row
        if constexpr (!kStates) {
            const int t = tid / (P / 8), c8 = tid % (P / 8);
            if (c0 + t < L)
                st_global16(yg + (c0 + t) * xrow + 8 * c8,
                            *reinterpret_cast<const u32x4 *>(Ys + t * SM::kPY + 8 * c8));
        }
        if (c + 1 < nch) stash_chunk(c0 + kQ);
        __syncthreads();
    }

    if (!kStates && p.last_state) {
        float *ls = p.last_state + ((b * H + h) * P + col) * N;
#pragma unroll
        for (int mm = 0; mm < kNH; mm++)
            *reinterpret_cast<f32x4 *>(ls + 16 * (m0 + mm) + 4 * lg) = Hs[mm];
    }
}

template <int N, bool kStates>
hipError_t launch_n(const SsdParams &p, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.batch * p.nheads));
    switch (p.headdim) {
        case 16: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 16, kStates>), grid, dim3(128), 0, stream, p); break;
        case 32: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 32, kStates>), grid, dim3(256), 0, stream, p); break;
        case 48: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 48, kStates>), grid, dim3(384), 0, stream, p); break;
        case 64: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 64, kStates>), grid, dim3(512), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

template <bool kStates>
hipError_t launch_any(const SsdParams &p, hipStream_t stream) {
    if (p.batch == 0 || p.nheads == 0) return hipSuccess;
    hipError_t e;
    switch (p.dstate) {
        case 32: e = launch_n<32, kStates>(p, stream); break;
        case 64: e = launch_n<64, kStates>(p, stream); break;
        case 96: e = launch_n<96, kStates>(p, stream); break;
        case 128: e = launch_n<128, kStates>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    profile_mark(stream);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace

hipError_t launch_ssd_fwd(const SsdParams &p, hipStream_t stream) {
    return launch_any<false>(p, stream);
}

hipError_t launch_ssd_states(const SsdParams &p, hipStream_t stream) {
    return launch_any<true>(p, stream);
}

size_t ssd_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                      int64_t dstate) {
    if (batch <= 0 || nheads <= 0 || seqlen <= 0) return 0;
    return size_t(batch) * size_t(nheads) * size_t((seqlen + kQ - 1) / kQ) * size_t(dstate) *
           size_t(headdim) * 4;
}

}  // namespace ssk
