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
//   Y += C H^T (over d_state; 16x16x32), H^T += B^T (w X) (over the chunk; 16x16x32).
//
// Work mapping.  One workgroup per (batch, head), four wavefronts per 16
// columns (see the kernel).  The state lives in MFMA accumulators as H^T
// tiles (16 states x 16 columns); their registers are, after the bf16
// split, exactly the B operand of the C H^T product.  G^T is computed
// (rather than G) because its accumulator registers, scaled by
// exp(cum_t - cum_s) dt_s, are the A operand of the W X product in the
// same lane layout; W does not depend on the column, so each W tile is made
// once per chunk and shared through LDS.  A chunk's B, C (row-major,
// d_state contiguous), B^T and x^T (time contiguous) and dt go through LDS;
// the next chunk is loaded into registers while the current one is
// computed.  The chunk's output is gathered in LDS and written in whole
// 16-byte pieces of full rows (a head's row is headdim contiguous values):
// 2-byte stores of a wavefront's 16 columns cost more than the rest of the
// kernel together.
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

// Inclusive running sum over the 64 lanes of a wavefront on DPP moves: shifts
// by 1, 2, 4 and 8 within each row of 16 lanes, then the last lane of row 0
// into row 1 (and of row 2 into row 3), then lane 31 into rows 2 and 3.
__device__ __forceinline__ float wave_incl_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));
    return x;
}

// LDS of one workgroup (the states pass keeps only B^T, x^T, the w x split
// and the running sums).
template <int N, int P, bool kStates>
struct SsdSmem {
    static constexpr int kPB = N + 8;   // row pitch of B and C (bf16), 16-byte multiple
    static constexpr int kPT = kQ + 8;  // row pitch of B^T, x^T and the w x split (bf16)
    static constexpr int kPY = P + 8;   // row pitch of the output tile (bf16)
    static constexpr int kNT = N / 16, kCT = P / 16;
    static constexpr uint32_t kRow = kStates ? 0 : kQ * kPB * 2;
    static constexpr uint32_t kBs = 0;                           // bf16 [kQ][kPB]
    static constexpr uint32_t kCs = kBs + kRow;                  // bf16 [kQ][kPB]
    static constexpr uint32_t kBT = kCs + kRow;                  // bf16 [N][kPT]
    static constexpr uint32_t kXT = kBT + N * kPT * 2;           // bf16 [2][P][kPT], by chunk parity
    static constexpr uint32_t kXSh = kXT + 2 * P * kPT * 2;      // bf16 [P][kPT]: hi part of w x
    static constexpr uint32_t kXSl = kXSh + P * kPT * 2;         // bf16 [P][kPT]: lo part of w x
    // f32 [2][4][kQ], by chunk parity: cum, dt, w = exp(cum_last - cum_s) dt_s, exp(cum)
    static constexpr uint32_t kScan = kXSl + P * kPT * 2;
    static constexpr uint32_t kYs = kScan + 2 * 4 * kQ * 4;      // bf16 [kQ][kPY]: the chunk's output
    static constexpr uint32_t kHx = kYs + (kStates ? 0 : kQ * kPY * 2);
    // state exchange: [column tile][state tile][lane] x 16 bytes (bf16 hi, lo)
    static constexpr uint32_t kWx = kHx + (kStates ? 0 : kCT * kNT * 64 * 16);
    // the chunk's ten lower-triangle W tiles: [tile][lane] x 16 bytes (bf16 hi, lo)
    static constexpr uint32_t kSize = kWx + (kStates ? 0 : 10 * 64 * 16);
};

// N: dstate (multiple of 32, <= 128); P: headdim (multiple of 16, <= 64).
// Sixteen wavefronts per 64 columns: wavefront (q, ti) owns the output
// tile of time tile ti (steps 16 ti .. 16 ti + 15 of the chunk) and column
// tile q (columns 16 q .. 16 q + 15), and carries the state tiles m = ti,
// ti + 4, ... of that column tile.  Per chunk, in two phases between two
// barriers:
//   phase 1: B^T of the chunk into LDS; the w x split; the ten W tiles
//     (G^T = B C^T scaled and masked; wavefront k makes tile k, so each is
//     made once for all columns); C H_in for the own output tile from the
//     published state; the previous chunk's output rows to memory;
//   phase 2: W x for the own tile, the output tile into LDS; the state
//     update of the own state tiles and their publication; B, C, x^T and
//     the running sums of the next chunk into LDS.
// Every buffer written in one phase was last read in the other (x^T and
// the running sums are read in both and are double-buffered), so two
// barriers per chunk suffice.
//
// The state entering chunk c is stored to p.states, when given, as (batch,
// head, chunk) blocks of a dstate x headdim f32 matrix (headdim contiguous):
// the forward's checkpoint for the backward.  kStates: the backward's own
// states pass, when no checkpoint was saved.  Only the recurrence runs (no
// output, no C H_in, no W x), with the same arithmetic, so the states are
// the same bits.
template <int N, int P, bool kStates>
__global__ __launch_bounds__(16 * P) void ss_ssd_fwd_kernel(SsdParams p) {
    constexpr int kCT = P / 16, kNT = N / 16;
    constexpr int kWaves = 4 * kCT, kThr = 64 * kWaves;
    constexpr int kNH = (kNT + 3) / 4;               // state tiles per wavefront, at most
    constexpr int kVB = kQ * N / 8;                  // 16-byte vectors of a B (or C) chunk
    constexpr int kBV = (kVB + kThr - 1) / kThr;     // per thread
    constexpr int kVX = kQ * P / 8;                  // 16-byte vectors of an x chunk
    static_assert(2 * kVX == kThr, "x vectors for half the threads");
    using SM = SsdSmem<N, P, kStates>;
    __shared__ __attribute__((aligned(16))) char smem[SM::kSize];
    bf16_t *Bs = reinterpret_cast<bf16_t *>(smem + SM::kBs);
    bf16_t *Cs = reinterpret_cast<bf16_t *>(smem + SM::kCs);
    bf16_t *BT = reinterpret_cast<bf16_t *>(smem + SM::kBT);
    bf16_t *XSh = reinterpret_cast<bf16_t *>(smem + SM::kXSh);
    bf16_t *XSl = reinterpret_cast<bf16_t *>(smem + SM::kXSl);
    bf16_t *Ys = reinterpret_cast<bf16_t *>(smem + SM::kYs);
    auto XT = [&](int buf) { return reinterpret_cast<bf16_t *>(smem + SM::kXT) + buf * P * SM::kPT; };
    auto scan = [&](int buf, int k) { return reinterpret_cast<float *>(smem + SM::kScan) + (buf * 4 + k) * kQ; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int q = wv % kCT, ti = wv / kCT;
    const int li = lane & 15, lg = lane >> 4;
    const int col = 16 * q + li;
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

    // state tile m = ti + 4 mm (when m < kNT): lane holds
    // H^T[n = 16 m + 4 lg + r][col]
    f32x4 Hs[kNH];
    if (p.h0) {   // one test for all loads, so they are issued together
        const float *h0 = p.h0 + ((b * H + h) * P + col) * N;
#pragma unroll
        for (int mm = 0; mm < kNH; mm++) {
            const int m = ti + 4 * mm;
            Hs[mm] = m < kNT ? *reinterpret_cast<const f32x4 *>(h0 + 16 * m + 4 * lg) : kZero4;
        }
    } else {
#pragma unroll
        for (int mm = 0; mm < kNH; mm++) Hs[mm] = kZero4;
    }
    auto hx = [&](int m) {
        return reinterpret_cast<s16x4 *>(smem + SM::kHx + ((q * kNT + m) * 64 + lane) * 16);
    };
    auto publish = [&]() {
#pragma unroll
        for (int mm = 0; mm < kNH; mm++) {
            const int m = ti + 4 * mm;
            if (m < kNT) {
                s16x4 hi, lo;
                split4(Hs[mm], hi, lo);
                s16x4 *e = hx(m);
                e[0] = hi;
                e[1] = lo;
            }
        }
    };

    // the next chunk, in registers
    u32x4 rb[kBV], rc[kBV], rx;
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
        if (tid < kVX) {
            const int s = tid % kQ, c8 = tid / kQ;
            const int64_t t = c0 + s < L ? c0 + s : L - 1;
            rx = ld_global16(xg + t * xrow + 8 * c8);
        }
    };
    // registers -> LDS (B and C rows, x^T, the running sums); steps past the
    // end become zeros (no input, no decay)
    auto stash_rows = [&](int64_t c0, int buf) {
        if constexpr (!kStates) {
#pragma unroll
            for (int k = 0; k < kBV; k++) {
                const int v = tid + k * kThr;
                if (v < kVB) {
                    const int s = v % kQ, c8 = v / kQ;
                    const bool live = c0 + s < L;
                    u32x4 vb = rb[k], vc = rc[k];
                    if (!live) vb = vc = u32x4{0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4 *>(Bs + s * SM::kPB + 8 * c8) = vb;
                    *reinterpret_cast<u32x4 *>(Cs + s * SM::kPB + 8 * c8) = vc;
                }
            }
        }
        if (tid < kVX) {
            const int s = tid % kQ, c8 = tid / kQ;
            u32x4 vx = rx;
            if (!(c0 + s < L)) vx = u32x4{0u, 0u, 0u, 0u};
            bf16_t *xt = XT(buf);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                xt[(8 * c8 + 2 * e) * SM::kPT + s] = bf16_t(vx[e] & 0xffffu);
                xt[(8 * c8 + 2 * e + 1) * SM::kPT + s] = bf16_t(vx[e] >> 16);
            }
        }
    };
    // dt of a chunk (raw bf16 bits, lane = step) -> dt, the running sum of
    // dt A, w and exp(cum), on the last wavefront, one chunk ahead of the
    // others (its dt is loaded two chunks ahead)
    constexpr int kScanWave = kWaves - 1;
    auto load_dt = [&](int64_t c0) {
        const int64_t t = c0 + lane < L ? c0 + lane : L - 1;
        return ld_global(dtg + t * H);
    };
    auto scan_dt = [&](int64_t c0, int buf, uint32_t raw) {
        float dv = 0.0f;
        if (c0 + lane < L) {
            dv = bf_lo(raw & 0xffffu) + bias;
            if (p.softplus) dv = softplus_f32(dv);
        }
        // running sum of dt A in base-2 exponent units (plain f32: the
        // rounding of large sums stays far below the bf16 output's; the
        // backward, whose dA needs more, carries it compensated)
        const float a = wave_incl_sum(dv * a2);
        const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 63));
        scan(buf, 0)[lane] = a;
        scan(buf, 1)[lane] = dv;
        scan(buf, 2)[lane] = exp2_hw(total - a) * dv;
        scan(buf, 3)[lane] = exp2_hw(a);
    };
    // registers -> B^T (the state update's operand)
    auto stash_bt = [&](int64_t c0) {
#pragma unroll
        for (int k = 0; k < kBV; k++) {
            const int v = tid + k * kThr;
            if (v < kVB) {
                const int s = v % kQ, c8 = v / kQ;
                u32x4 vb = rb[k];
                if (!(c0 + s < L)) vb = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    BT[(8 * c8 + 2 * e) * SM::kPT + s] = bf16_t(vb[e] & 0xffffu);
                    BT[(8 * c8 + 2 * e + 1) * SM::kPT + s] = bf16_t(vb[e] >> 16);
                }
            }
        }
    };
    // a chunk's output rows: 16-byte stores, P / 8 lanes per row
    // (the second half of the threads: the first wavefronts make the W tiles
    // in the same phase)
    auto store_rows = [&](int64_t c0) {
        const int i = tid - (kThr - kQ * P / 8);
        const int t = i / (P / 8), c8 = i % (P / 8);
        if (i >= 0 && c0 + t < L)
            st_global16(yg + (c0 + t) * xrow + 8 * c8,
                        *reinterpret_cast<const u32x4 *>(Ys + t * SM::kPY + 8 * c8));
    };

    const int64_t nch = (L + kQ - 1) / kQ;
    if constexpr (!kStates) publish();
    uint32_t rdt = 0;   // dt of chunk c + 1, on the scan wavefront
    if (nch > 0) {
        load_chunk(0);
        if (wv == kScanWave) {
            scan_dt(0, 0, load_dt(0));
            if (nch > 1) rdt = load_dt(kQ);
        }
        stash_rows(0, 0);
    }
    __syncthreads();
    for (int64_t c = 0; c < nch; c++) {
        const int64_t c0 = c * kQ;
        const int buf = int(c & 1);
        const bf16_t *xt = XT(buf);
        const float *cum = scan(buf, 0);
        // ---------------- phase 1
        stash_bt(c0);
        if (c + 1 < nch) load_chunk(c0 + kQ);
        if (wv == kScanWave && c + 1 < nch) {
            // the next chunk's sums (their buffer was last read by chunk c - 1)
            scan_dt(c0 + kQ, buf ^ 1, rdt);
            if (c + 2 < nch) rdt = load_dt(c0 + 2 * kQ);
        }
        if constexpr (!kStates) {
            if (c > 0) store_rows(c0 - kQ);
        }
        if (kStates || p.states) {
            // H_in of this chunk: lane holds H^T[n][col], 16 lanes one row piece
            float *st = p.states + (((b * H + h) * nch + c) * N) * P + col;
#pragma unroll
            for (int mm = 0; mm < kNH; mm++) {
                const int m = ti + 4 * mm;
                if (m < kNT) {
#pragma unroll
                    for (int r = 0; r < 4; r++) st[(16 * m + 4 * lg + r) * P] = Hs[mm][r];
                }
            }
        }
        // w x as bf16 high and low parts, two steps of one column per pair
        {
            const float *wts = scan(buf, 2);
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int v = tid + k * kThr;
                const int cc = v / (kQ / 2), s = 2 * (v % (kQ / 2));
                const uint32_t xr = *reinterpret_cast<const uint32_t *>(xt + cc * SM::kPT + s);
                uint32_t hw, lw;
                split2(bf_lo(xr) * wts[s], bf_hi(xr) * wts[s + 1], hw, lw);
                *reinterpret_cast<uint32_t *>(XSh + cc * SM::kPT + s) = hw;
                *reinterpret_cast<uint32_t *>(XSl + cc * SM::kPT + s) = lw;
            }
        }
        f32x4 Y = kZero4;
        if constexpr (!kStates) {
            const float *dts = scan(buf, 1);
            // W tile k = (i, j), j <= i: W[t = 16 i + li][s = 16 j + 4 lg + r]
            // = G^T[s][t] exp(cum_t - cum_s) dt_s, s <= t
            for (int k = wv; k < 10; k += kWaves) {
                const int i = k >= 6 ? 3 : k >= 3 ? 2 : k >= 1 ? 1 : 0;
                const int j = k - i * (i + 1) / 2;
                const int t = 16 * i + li;
                const float ct = cum[t];
                const f32x4 cs = *reinterpret_cast<const f32x4 *>(cum + 16 * j + 4 * lg);
                const f32x4 ds = *reinterpret_cast<const f32x4 *>(dts + 16 * j + 4 * lg);
                bf16x8_t cb[N / 32], ba[N / 32];
#pragma unroll
                for (int kk = 0; kk < N / 32; kk++) {
                    cb[kk] = *reinterpret_cast<const bf16x8_t *>(Cs + t * SM::kPB + 32 * kk + 8 * lg);
                    ba[kk] = *reinterpret_cast<const bf16x8_t *>(Bs + (16 * j + li) * SM::kPB + 32 * kk + 8 * lg);
                }
                f32x4 gt = kZero4;   // G^T[s = 16 j + 4 lg + r][t]
#pragma unroll
                for (int kk = 0; kk < N / 32; kk++) gt = mfma32(ba[kk], cb[kk], gt);
                f32x4 w;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    w[r] = gt[r] * exp2_hw(ct - cs[r]) * ds[r];
                    // below the diagonal s < t always; on it keep s <= t
                    if (i == j) w[r] = (4 * lg + r <= li) ? w[r] : 0.0f;
                }
                s16x4 wh, wl;
                split4(w, wh, wl);
                s16x4 *e = reinterpret_cast<s16x4 *>(smem + SM::kWx + (k * 64 + lane) * 16);
                e[0] = wh;
                e[1] = wl;
            }
            // C H_in for time tile ti: the 16x16x32 product runs over state
            // tiles 2 m2 and 2 m2 + 1 at once, its k index over (tile, 4 lg +
            // r) in the order the state accumulators hold them, and C is read
            // in that same order
            const bf16_t *crow = Cs + (16 * ti + li) * SM::kPB + 4 * lg;
            // (the high and low parts in two accumulators: two independent
            // chains of products, added at the end)
            f32x4 Ylo = kZero4;
#pragma unroll
            for (int m2 = 0; m2 < kNT / 2; m2++) {
                const s16x4 *e0 = hx(2 * m2), *e1 = hx(2 * m2 + 1);
                const bf16x8_t a = cat8(*reinterpret_cast<const s16x4 *>(crow + 32 * m2),
                                        *reinterpret_cast<const s16x4 *>(crow + 32 * m2 + 16));
                Y = mfma32(a, cat8(e0[0], e1[0]), Y);
                Ylo = mfma32(a, cat8(e0[1], e1[1]), Ylo);
            }
            const f32x4 ec = *reinterpret_cast<const f32x4 *>(scan(buf, 3) + 16 * ti + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; r++) Y[r] = (Y[r] + Ylo[r]) * ec[r];
        }
        __syncthreads();
        // ---------------- phase 2
        if constexpr (!kStates) {
            // Y += W x over the tiles j <= ti (x[s][col] as the B operand)
            s16x4 xb[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                if (j <= ti) xb[j] = *reinterpret_cast<const s16x4 *>(xt + col * SM::kPT + 16 * j + 4 * lg);
            f32x4 Ylo = kZero4;   // the low parts' products, a chain of their own
#pragma unroll
            for (int j = 0; j < 4; j++) {
                if (j <= ti) {
                    const s16x4 *e = reinterpret_cast<const s16x4 *>(
                        smem + SM::kWx + ((ti * (ti + 1) / 2 + j) * 64 + lane) * 16);
                    Y = mfma16(e[0], xb[j], Y);
                    Ylo = mfma16(e[1], xb[j], Ylo);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; r++) Y[r] += Ylo[r];
            // y + D x into the output tile (lane holds y[t = 16 ti + 4 lg + r][col];
            // x at these steps is xb[ti], two values per dword); it leaves in
            // whole rows in the next phase 1
            s16x4 xo = xb[0];
#pragma unroll
            for (int j = 1; j < 4; j++)
                if (j == ti) xo = xb[j];
            const u32x2_t xw = __builtin_bit_cast(u32x2_t, xo);
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int t = 16 * ti + 4 * lg + 2 * k;
                const uint32_t yv = pk_bf16(Y[2 * k] + dskip * bf_lo(xw[k]),
                                            Y[2 * k + 1] + dskip * bf_hi(xw[k]));
                Ys[t * SM::kPY + col] = bf16_t(yv & 0xffffu);
                Ys[(t + 1) * SM::kPY + col] = bf16_t(yv >> 16);
            }
        }
        // the own state tiles: H_out = exp(cum_last) H_in + B^T (w x)
        {
            const float decay = exp2_hw(cum[kQ - 1]);
            bf16x8_t xsh[2], xsl[2];
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                xsh[kk] = *reinterpret_cast<const bf16x8_t *>(XSh + col * SM::kPT + 32 * kk + 8 * lg);
                xsl[kk] = *reinterpret_cast<const bf16x8_t *>(XSl + col * SM::kPT + 32 * kk + 8 * lg);
            }
#pragma unroll
            for (int mm = 0; mm < kNH; mm++) {
                const int m = ti + 4 * mm;
                if (m < kNT) {
#pragma unroll
                    for (int r = 0; r < 4; r++) Hs[mm][r] *= decay;
#pragma unroll
                    for (int kk = 0; kk < 2; kk++) {
                        const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(BT + (16 * m + li) * SM::kPT + 32 * kk + 8 * lg);
                        Hs[mm] = mfma32(a, xsh[kk], Hs[mm]);
                        Hs[mm] = mfma32(a, xsl[kk], Hs[mm]);
                    }
                }
            }
        }
        if constexpr (!kStates) publish();
        if (c + 1 < nch) stash_rows(c0 + kQ, buf ^ 1);
        __syncthreads();
    }
    if constexpr (!kStates) {
        if (nch > 0) store_rows((nch - 1) * kQ);
    }

    if (!kStates && p.last_state) {
        float *ls = p.last_state + ((b * H + h) * P + col) * N;
#pragma unroll
        for (int mm = 0; mm < kNH; mm++) {
            const int m = ti + 4 * mm;
            if (m < kNT) *reinterpret_cast<f32x4 *>(ls + 16 * m + 4 * lg) = Hs[mm];
        }
    }
}

template <int N, bool kStates>
hipError_t launch_n(const SsdParams &p, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.batch * p.nheads));
    switch (p.headdim) {
        case 16: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 16, kStates>), grid, dim3(256), 0, stream, p); break;
        case 32: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 32, kStates>), grid, dim3(512), 0, stream, p); break;
        case 48: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 48, kStates>), grid, dim3(768), 0, stream, p); break;
        case 64: hipLaunchKernelGGL((ss_ssd_fwd_kernel<N, 64, kStates>), grid, dim3(1024), 0, stream, p); break;
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
