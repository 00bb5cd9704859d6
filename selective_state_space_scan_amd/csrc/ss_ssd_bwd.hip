// ss_ssd_bwd.hip -- Mamba-2 SSD backward in chunked form on gfx950 matrix cores.
//
// The forward (ss_ssd.hip; the SSD module that the state-spaces/mamba README
// names under "Mamba-2") is, per batch b and head h, with dt_t after bias and
// softplus, a_t = dt_t A[h] and cum_t the running sum of a over a chunk of
// kQ = 64 steps,
//   y_t   = exp(cum_t) H_in C_t + sum_{s<=t} exp(cum_t - cum_s) (C_t . B_s) dt_s x_s + D x_t
//   H_out = exp(cum_last) H_in  + sum_s exp(cum_last - cum_s) dt_s x_s B_s^T.
// Back-propagation through time, regrouped by chunk.  With dH = dL/dH_out
// of the chunk, L_ts = exp(cum_t - cum_s) (s <= t, else 0), G_ts = C_t . B_s,
// M_ts = dy_t . x_s, wB_s = exp(cum_last - cum_s):
//   dx_s   = sum_t G_ts L_ts dt_s dy_t + dt_s wB_s dH B_s + D dy_s
//   dC_t   = sum_s (M_ts L_ts dt_s) B_s + exp(cum_t) H_in^T dy_t
//   dB_s   = sum_t (M_ts L_ts dt_s) C_t + dt_s wB_s dH^T x_s
//   dH_in  = exp(cum_last) dH + sum_t exp(cum_t) dy_t C_t^T
// and, through dt directly (u) and through the running sums (v, the
// gradient w.r.t. cum_t; the gradient w.r.t. a_s is then sum_{t>=s} v_t):
//   u_s = sum_t G_ts L_ts M_ts + q_s,  q_s = wB_s x_s^T dH B_s
//   v_t = sum_s G_ts L_ts M_ts dt_s - dt_t u_t + exp(cum_t) dy_t^T H_in C_t
//         (+ exp(cum_last) <dH, H_in> + sum_s dt_s q_s at the last step)
//   d(dt_s) = u_s + A sum_{t>=s} v_t,  dA = sum_s dt_s sum_{t>=s} v_t.
//
// Kernels, in order:
//   1. states pass (ss_ssd.hip): H_in of every chunk, f32, to the workspace
//      (skipped when the forward saved them: ckpt);
//   2. ss_ssd_bwd_kernel: one workgroup per (batch, head) walks the chunks
//      last to first with dH in matrix-core accumulators; writes dx, the
//      head's dB and dC terms (f32, per head), u and v per step, and dh0;
//   3. ssd_bwd_dt_kernel: per chunk, the suffix sums of v, ddt, and the
//      chunk's dA and ddt_bias terms;
//   4. ssd_bwd_fold_kernel: dB and dC summed over the heads of a group;
//   5. ssd_bwd_param_kernel: dA, dD, ddt_bias summed over batch and chunks.
// Every sum runs in a fixed order: results are bit-reproducible and do not
// depend on the batch size.
//
// Rounding: x, dy, B, C are bf16 already.  Operands made on chip (the W and
// dGm tiles, H_in, dH, exp(cum) dy) are split into a bf16 high and low part
// and multiplied as two products, as in the forward; sums are f32.  dA is
// the exception that needs more: it is a sum over the chunk of suffix sums
// in which large terms cancel.  So the running sums of dt A are carried as
// compensated hi + lo pairs, the per-step sums that build v (and dA itself)
// are f64, and dH and H_in enter the products behind q and r in three bf16
// parts (2^-27).
#include <type_traits>

#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_mfma.h"
#include "ss_tiles.h"

namespace ssk {
namespace {

constexpr int kQ = 64;  // chunk length
constexpr int kWaves = 8, kThr = 64 * kWaves;

struct BwdWs {
    float *states;     // (batch, head, chunk, dstate, headdim): H_in
    float *pdB, *pdC;  // (batch, head, chunk, time tile, state tile, lane, 4): per-head terms
    float *u;          // (batch, head, chunk, kQ)
    double *v;         // (batch, head, chunk, kQ)
    double *dAp;       // (batch, head, chunk)
    float *dbp;        // (batch, head, chunk)
    float *dDp;        // (batch, head)
};

BwdWs carve(void *base, int64_t batch, int64_t nheads, int64_t nch, int64_t P, int64_t N,
            size_t *total) {
    BwdWs w{};
    size_t off = 0;
    char *b = static_cast<char *>(base);
    auto take = [&](auto **dst, int64_t count) {
        using T = std::remove_reference_t<decltype(**dst)>;
        *dst = base ? reinterpret_cast<T *>(b + off) : nullptr;
        off += (size_t(count) * sizeof(T) + 255) / 256 * 256;
    };
    const int64_t bhc = batch * nheads * nch;
    take(&w.states, bhc * N * P);
    take(&w.pdB, bhc * kQ * N);
    take(&w.pdC, bhc * kQ * N);
    take(&w.u, bhc * kQ);
    take(&w.v, bhc * kQ);
    take(&w.dAp, bhc);
    take(&w.dbp, bhc);
    take(&w.dDp, batch * nheads);
    if (total) *total = off;
    return w;
}

template <int N, int P>
struct BwdSmem {
    static constexpr int kPB = N + 8;   // row pitch of B, C (bf16)
    static constexpr int kPT = kQ + 8;  // row pitch of B^T, C^T, dy^T (bf16)
    static constexpr int kPX = P + 8;   // row pitch of x, dy, dx (bf16)
    static constexpr int kPH = P + 4;   // row pitch of dH stored [n][p] (f32)
    static constexpr uint32_t kBs = 0;
    static constexpr uint32_t kCs = kBs + kQ * kPB * 2;
    static constexpr uint32_t kBT = kCs + kQ * kPB * 2;
    static constexpr uint32_t kCT = kBT + N * kPT * 2;
    static constexpr uint32_t kXs = kCT + N * kPT * 2;
    static constexpr uint32_t kYs = kXs + kQ * kPX * 2;
    static constexpr uint32_t kYT = kYs + kQ * kPX * 2;
    static constexpr uint32_t kHf = kYT + P * kPT * 2;   // f32 [N][kPH]: dH of the chunk's end
    static constexpr uint32_t kDX = kHf + N * kPH * 4;
    static constexpr uint32_t kCum = kDX + kQ * kPX * 2;  // f32: running sum of dt A, base 2
    static constexpr uint32_t kDt = kCum + kQ * 4;        // f32: dt
    static constexpr uint32_t kEc = kDt + kQ * 4;         // f32: exp(cum_t)
    static constexpr uint32_t kWb = kEc + kQ * 4;         // f32: exp(cum_last - cum_s)
    static constexpr uint32_t kUg = kWb + kQ * 4;         // f64 [8][kQ]: sum_t G L M per wavefront
    static constexpr uint32_t kVr = kUg + 8 * kQ * 8;     // f64 [8][kQ]: sum_s G L M dt_s per wavefront
    static constexpr uint32_t kQa = kVr + 8 * kQ * 8;     // f32 [8][kQ]: q terms per wavefront
    static constexpr uint32_t kRa = kQa + 8 * kQ * 4;     // f32 [8][kQ]: H_in terms per wavefront
    static constexpr uint32_t kHd = kRa + 8 * kQ * 4;     // f32 [8]: <dH, H_in> per wavefront
    static constexpr uint32_t kCumLo = kHd + 8 * 4;       // f32: low part of the running sum
    static constexpr uint32_t kSize = kCumLo + kQ * 4;
};

// Lane exchanges on DPP moves and lane swaps (no LDS round trips).  A DPP
// move of a 32-bit value; rotations within a row and quad permutations read
// a lane of the same row, so every lane has a source.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}
constexpr int kRor8 = 0x128, kRor4 = 0x124, kXor2 = 0x4E, kXor1 = 0xB1, kHalfMirror = 0x141;

// v_permlane32_swap with both operands v hands lane i the value of lane
// i ^ 32 in its second result; v_permlane16_swap pairs rows 0-1 and 2-3 the
// same way.  The two results are added in the same order in both lanes.
__device__ __forceinline__ float half_swap_sum(float v, bool rows) {
    const unsigned x = __float_as_uint(v);
    const auto r = rows ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                        : __builtin_amdgcn_permlane32_swap(x, x, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __uint_as_float(r0) + __uint_as_float(r1);
}
__device__ __forceinline__ double half_swap_sumd(double v, bool rows) {
    const unsigned lo = unsigned(__double2loint(v)), hi = unsigned(__double2hiint(v));
    const auto rl = rows ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                         : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto rh = rows ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                         : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const unsigned l0 = rl[0], l1 = rl[1], h0 = rh[0], h1 = rh[1];
    return __hiloint2double(int(h0), int(l0)) + __hiloint2double(int(h1), int(l1));
}

// Sum over the 16 lanes of a row, the same bits in every lane: lanes 8
// apart, then 4 apart (rotations, so each pair is added in one order in both
// of its lanes), then within quads.
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f<kRor8>(v);
    v += dpp_f<kRor4>(v);
    v += dpp_f<kXor2>(v);
    v += dpp_f<kXor1>(v);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    v = sum16(v);
    v = half_swap_sum(v, false);
    return half_swap_sum(v, true);
}

__device__ __forceinline__ double sum16d(double v) {
    v += dpp_d<kRor8>(v);
    v += dpp_d<kRor4>(v);
    v += dpp_d<kXor2>(v);
    v += dpp_d<kXor1>(v);
    return v;
}

__device__ __forceinline__ double wave_sumd(double v) {
    v = sum16d(v);
    v = half_swap_sumd(v, false);
    return half_swap_sumd(v, true);
}

// Sums of four values over the 16 lanes of a row, scattered: lane li gets
// the sum of x[li / 4 % 4].  Five exchanges (two, then one per level) in
// place of four full butterflies: lanes 8 apart (li ^ 8, a rotation by 8),
// then across the two quads of each half row (a mirror within the half: a
// lane reads a different lane of the other quad than li ^ 4, which the quad
// sums after it do not notice), then within quads.
template <typename T, int CTRL>
__device__ __forceinline__ T dpp_any(T v) {
    if constexpr (sizeof(T) == 8) return dpp_d<CTRL>(v);
    else return dpp_f<CTRL>(v);
}
template <typename T>
__device__ __forceinline__ T sum16x4(const T (&x)[4], int li) {
    const bool b3 = li & 8, b2 = li & 4;
    const T y0 = (b3 ? x[2] : x[0]) + dpp_any<T, kRor8>(b3 ? x[0] : x[2]);
    const T y1 = (b3 ? x[3] : x[1]) + dpp_any<T, kRor8>(b3 ? x[1] : x[3]);
    T z = (b2 ? y1 : y0) + dpp_any<T, kHalfMirror>(b2 ? y0 : y1);
    z += dpp_any<T, kXor2>(z);
    z += dpp_any<T, kXor1>(z);
    return z;
}

__device__ __forceinline__ float pick4(const float (&v)[4], int k) {
    return k == 0 ? v[0] : k == 1 ? v[1] : k == 2 ? v[2] : v[3];
}

// One workgroup of 8 wavefronts per (batch, head).  Wavefront wv = 2 sg + cls.
// Class cls owns time tiles {0, 3} (cls 0) or {1, 2} (cls 1) -- as s tiles of
// the dx and dB products and as t tiles of the dC product, five of the ten
// lower-triangle tiles each -- and sg splits the columns: dx column tile sg,
// state tiles sg, sg + 4; the per-step sums of a class's tiles are split by
// rows (wavefront sg adds rows 4 lg + sg).  The carried dH^T tiles k = wv +
// 8 kk (state tile k / (P / 16), column tile k % (P / 16)) are spread over
// all wavefronts and published in LDS as an f32 [state][column] matrix each
// chunk, split into bf16 parts where it is used.
template <int N, int P>
__global__ __launch_bounds__(kThr) void ss_ssd_bwd_kernel(SsdBwdParams p, BwdWs ws) {
    constexpr int kCT = P / 16, kNT = N / 16;
    constexpr int kVB = kQ * N / 8;                      // 16-byte vectors of a B (or C) chunk
    constexpr int kBV = (kVB + kThr - 1) / kThr;
    constexpr int kVX = kQ * P / 8;                      // 16-byte vectors of an x (or dy) chunk
    static_assert(kVX <= kThr, "one x vector per thread at most");
    constexpr int kDH = (kNT * kCT + kWaves - 1) / kWaves;   // dH tiles per wavefront
    constexpr int kNS = (kNT + 3) / 4;                   // state tiles per wavefront
    using SM = BwdSmem<N, P>;
    __shared__ __attribute__((aligned(16))) char smem[SM::kSize];
    bf16_t *Bs = reinterpret_cast<bf16_t *>(smem + SM::kBs);
    bf16_t *Cs = reinterpret_cast<bf16_t *>(smem + SM::kCs);
    bf16_t *BT = reinterpret_cast<bf16_t *>(smem + SM::kBT);
    bf16_t *CT = reinterpret_cast<bf16_t *>(smem + SM::kCT);
    bf16_t *Xs = reinterpret_cast<bf16_t *>(smem + SM::kXs);
    bf16_t *Ys = reinterpret_cast<bf16_t *>(smem + SM::kYs);
    bf16_t *YT = reinterpret_cast<bf16_t *>(smem + SM::kYT);
    float *Hf = reinterpret_cast<float *>(smem + SM::kHf);
    bf16_t *DX = reinterpret_cast<bf16_t *>(smem + SM::kDX);
    float *cum = reinterpret_cast<float *>(smem + SM::kCum);
    float *cumlo = reinterpret_cast<float *>(smem + SM::kCumLo);
    float *dts = reinterpret_cast<float *>(smem + SM::kDt);
    float *ecum = reinterpret_cast<float *>(smem + SM::kEc);
    float *wbs = reinterpret_cast<float *>(smem + SM::kWb);
    double *Ug = reinterpret_cast<double *>(smem + SM::kUg);
    double *Vr = reinterpret_cast<double *>(smem + SM::kVr);
    float *Qa = reinterpret_cast<float *>(smem + SM::kQa);
    float *Ra = reinterpret_cast<float *>(smem + SM::kRa);
    float *Hd = reinterpret_cast<float *>(smem + SM::kHd);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int cls = wv & 1, sg = wv >> 1;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t H = p.nheads, G = p.ngroups, L = p.seqlen;
    const int64_t b = blockIdx.x % p.batch, h = blockIdx.x / p.batch;
    const int64_t g = h / (H / G), bh = b * H + h;
    const int64_t nch = (L + kQ - 1) / kQ;
    const float a2 = p.A[h] * kLog2e;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const float dskip = p.D ? p.D[h] : 0.0f;
    const int64_t xrow = H * P, brow = G * N;
    const bf16_t *xg = static_cast<const bf16_t *>(p.x) + (b * L * H + h) * P;
    const bf16_t *yg = static_cast<const bf16_t *>(p.dout) + (b * L * H + h) * P;
    const bf16_t *dtg = static_cast<const bf16_t *>(p.dt) + b * L * H + h;
    const bf16_t *Bg = static_cast<const bf16_t *>(p.B) + (b * L * G + g) * N;
    const bf16_t *Cg = static_cast<const bf16_t *>(p.C) + (b * L * G + g) * N;
    bf16_t *dxg = static_cast<bf16_t *>(p.dx) + (b * L * H + h) * P;
    const float *hin_g = ws.states + bh * nch * N * P;
    float *pdB = ws.pdB + bh * nch * kQ * N, *pdC = ws.pdC + bh * nch * kQ * N;
    float *ug = ws.u + bh * nch * kQ;
    double *vg = ws.v + bh * nch * kQ;

    // carried dH^T tiles: lane holds dH^T[n = 16 nt + 4 lg + r][p = 16 q + li]
    f32x4 dH[kDH];
#pragma unroll
    for (int kk = 0; kk < kDH; kk++) {
        const int k = wv + kWaves * kk;
        dH[kk] = kZero4;
        if (k < kNT * kCT && p.dlast) {
            const int nt = k / kCT, q = k % kCT;
            dH[kk] = *reinterpret_cast<const f32x4 *>(p.dlast + (bh * P + 16 * q + li) * N +
                                                     16 * nt + 4 * lg);
        }
    }
    auto publish = [&]() {
#pragma unroll
        for (int kk = 0; kk < kDH; kk++) {
            const int k = wv + kWaves * kk;
            if (k < kNT * kCT) {
                const int nt = k / kCT, q = k % kCT;
#pragma unroll
                for (int r = 0; r < 4; r++) Hf[(16 * nt + 4 * lg + r) * SM::kPH + 16 * q + li] = dH[kk][r];
            }
        }
    };

    // the next chunk (in time: the previous one), in registers
    u32x4 rb[kBV], rc[kBV], rx = {0u, 0u, 0u, 0u}, ry = {0u, 0u, 0u, 0u};
    uint32_t rdt = 0;
    // vector v of a chunk: 8 values of step s = v % kQ from value 8 (v / kQ)
    // on, so 64 lanes take 64 consecutive steps (conflict-free transposes)
    auto load_chunk = [&](int64_t c0) {
#pragma unroll
        for (int k = 0; k < kBV; k++) {
            const int v = tid + k * kThr;
            if (v < kVB) {
                const int s = v % kQ, c8 = v / kQ;
                const int64_t t = c0 + s < L ? c0 + s : L - 1;
                rb[k] = ld_global16(Bg + t * brow + 8 * c8);
                rc[k] = ld_global16(Cg + t * brow + 8 * c8);
            }
        }
        if (tid < kVX) {
            const int s = tid % kQ, c8 = tid / kQ;
            const int64_t t = c0 + s < L ? c0 + s : L - 1;
            rx = ld_global16(xg + t * xrow + 8 * c8);
            ry = ld_global16(yg + t * xrow + 8 * c8);
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
                u32x4 vb = rb[k], vc = rc[k];
                if (!live) vb = vc = u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4 *>(Bs + s * SM::kPB + 8 * c8) = vb;
                *reinterpret_cast<u32x4 *>(Cs + s * SM::kPB + 8 * c8) = vc;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    BT[(8 * c8 + 2 * e) * SM::kPT + s] = bf16_t(vb[e] & 0xffffu);
                    BT[(8 * c8 + 2 * e + 1) * SM::kPT + s] = bf16_t(vb[e] >> 16);
                    CT[(8 * c8 + 2 * e) * SM::kPT + s] = bf16_t(vc[e] & 0xffffu);
                    CT[(8 * c8 + 2 * e + 1) * SM::kPT + s] = bf16_t(vc[e] >> 16);
                }
            }
        }
        if (tid < kVX) {
            const int s = tid % kQ, c8 = tid / kQ;
            u32x4 vx = rx, vy = ry;
            if (!(c0 + s < L)) vx = vy = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(Xs + s * SM::kPX + 8 * c8) = vx;
            *reinterpret_cast<u32x4 *>(Ys + s * SM::kPX + 8 * c8) = vy;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                YT[(8 * c8 + 2 * e) * SM::kPT + s] = bf16_t(vy[e] & 0xffffu);
                YT[(8 * c8 + 2 * e + 1) * SM::kPT + s] = bf16_t(vy[e] >> 16);
            }
        }
        if (tid < kQ) {   // wavefront 0: dt, the running sum of dt A and its exponentials
            float dv = 0.0f;
            if (c0 + tid < L) {
                dv = bf_lo(rdt & 0xffffu) + bias;
                if (p.softplus) dv = softplus_f32(dv);
            }
            float a, alo;   // running sum of dt A in base-2 exponent units, hi + lo
            running_sum2(dv * a2, lane, a, alo);
            const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 63));
            const float tlo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alo), 63));
            cum[tid] = a;
            cumlo[tid] = alo;
            dts[tid] = dv;
            ecum[tid] = exp2_hw(a + alo);
            wbs[tid] = exp2_hw((total - a) + (tlo - alo));
        }
    };

    // 16 x 16 tile of U V^T over the headdim, U and V row tiles (at rows u0,
    // v0) of two [kQ][kPX] LDS arrays: 16x16x32 products when the headdim
    // allows, 16-byte operand reads (li_, lg_: the caller's lane index)
    auto rows_dot = [&](const bf16_t *U, int u0, const bf16_t *V, int v0, int li_, int lg_) {
        f32x4 acc = kZero4;
        if constexpr (P % 32 == 0) {
#pragma unroll
            for (int k = 0; k < P / 32; k++) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(U + (u0 + li_) * SM::kPX + 32 * k + 8 * lg_);
                const bf16x8_t bb = *reinterpret_cast<const bf16x8_t *>(V + (v0 + li_) * SM::kPX + 32 * k + 8 * lg_);
                acc = mfma32(a, bb, acc);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < kCT; kk++) {
                const s16x4 a = *reinterpret_cast<const s16x4 *>(U + (u0 + li_) * SM::kPX + 16 * kk + 4 * lg_);
                const s16x4 bb = *reinterpret_cast<const s16x4 *>(V + (v0 + li_) * SM::kPX + 16 * kk + 4 * lg_);
                acc = mfma16(a, bb, acc);
            }
        }
        return acc;
    };

    float dd = 0.0f;   // sum of dy . x over the class tiles' diagonals (used from sg == 0)

    // One chunk for this wavefront; HF = cls as a compile-time constant.
    auto chunk = [&](auto hfc, int64_t c) {
        constexpr int HF = decltype(hfc)::value;
        // The lane index, opaque to the compiler once per chunk: the LDS
        // addresses below are then computed inside the loop instead of being
        // hoisted out of it, where a hundred of them would stay live (and
        // spill) across every chunk.
        int lane_o = lane;
        asm volatile("" : "+v"(lane_o));
        const int li = lane_o & 15, lg = lane_o >> 4;
        constexpr int kT[2] = {HF ? 1 : 0, HF ? 2 : 3};
        // (t tile, s tile) pairs, s <= t: with the s tile in kT (kPi, kPj) and
        // with the t tile in kT (kRi, kRj)
        constexpr int kPi[5] = {HF ? 1 : 0, HF ? 2 : 1, HF ? 3 : 2, HF ? 2 : 3, 3};
        constexpr int kPj[5] = {HF ? 1 : 0, HF ? 1 : 0, HF ? 1 : 0, HF ? 2 : 0, HF ? 2 : 3};
        constexpr int kRi[5] = {HF ? 1 : 0, HF ? 1 : 3, HF ? 2 : 3, HF ? 2 : 3, HF ? 2 : 3};
        constexpr int kRj[5] = {0, HF ? 1 : 0, HF ? 0 : 1, HF ? 1 : 2, HF ? 2 : 3};
        const float elast = ecum[kQ - 1];

        // ---- dH^T <- exp(cum_last) dH^T + C^T (exp(cum) dy), this wavefront's tiles
#pragma unroll
        for (int kk = 0; kk < kDH; kk++) {
            const int k = wv + kWaves * kk;
            if (k < kNT * kCT) {
                const int nt = k / kCT, q = k % kCT;
                f32x4 acc = dH[kk];
#pragma unroll
                for (int r = 0; r < 4; r++) acc[r] *= elast;
#pragma unroll
                for (int k2 = 0; k2 < kQ / 32; k2++) {
                    const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(CT + (16 * nt + li) * SM::kPT + 32 * k2 + 8 * lg);
                    const u32x4 yr = *reinterpret_cast<const u32x4 *>(YT + (16 * q + li) * SM::kPT + 32 * k2 + 8 * lg);
                    const f32x4 e0 = *reinterpret_cast<const f32x4 *>(ecum + 32 * k2 + 8 * lg);
                    const f32x4 e1 = *reinterpret_cast<const f32x4 *>(ecum + 32 * k2 + 8 * lg + 4);
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float ea = e < 2 ? e0[2 * e] : e1[2 * e - 4];
                        const float eb = e < 2 ? e0[2 * e + 1] : e1[2 * e - 3];
                        split2(bf_lo(yr[e]) * ea, bf_hi(yr[e]) * eb, hw[e], lw[e]);
                    }
                    const bf16x8_t bh = bf16x8_of(hw[0], hw[1], hw[2], hw[3]);
                    const bf16x8_t bl = bf16x8_of(lw[0], lw[1], lw[2], lw[3]);
                    acc = mfma32(a, bh, acc);
                    acc = mfma32(a, bl, acc);
                }
                dH[kk] = acc;
            }
        }

        __builtin_amdgcn_sched_barrier(0);
        // ---- the dH parts of dx and dB for s tiles kT (lane: s = 16 j + 4 lg + r):
        // dx = dt_s wB_s B dH^T + D dy (column tile sg), dB = dt_s wB_s x dH
        // (state tiles sg + 4 ks), and q_s = wB_s sum_n B[s][n] (x dH)[s][n]
        const bool has_dx = sg < kCT;
        f32x4 dxa[2] = {kZero4, kZero4}, dba[2][kNS];
        if (has_dx) {
            const int q = sg;
#pragma unroll
            for (int k = 0; k < N / 32; k++) {
                // dH^T[n = 32 k + 8 lg + e][p = 16 q + li]: a column of the [n][p] store
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    split2(Hf[(32 * k + 8 * lg + 2 * e) * SM::kPH + 16 * q + li],
                           Hf[(32 * k + 8 * lg + 2 * e + 1) * SM::kPH + 16 * q + li], hw[e], lw[e]);
                const bf16x8_t hb = bf16x8_of(hw[0], hw[1], hw[2], hw[3]);
                const bf16x8_t lb = bf16x8_of(lw[0], lw[1], lw[2], lw[3]);
#pragma unroll
                for (int jj = 0; jj < 2; jj++) {
                    const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(Bs + (16 * kT[jj] + li) * SM::kPB + 32 * k + 8 * lg);
                    dxa[jj] = mfma32(a, hb, dxa[jj]);
                    dxa[jj] = mfma32(a, lb, dxa[jj]);
                }
                // one k step of 2-byte column reads at a time (registers)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // x dH for both s tiles, each dH operand split once: dH[p = 16 kk +
        // 4 lg + e][n = 16 nt + li] in three parts (q is summed over the chunk
        // for dA, where two-part rounding would show)
#pragma unroll
        for (int ks = 0; ks < kNS; ks++) {
            const int nt = sg + 4 * ks;
            dba[0][ks] = kZero4;
            dba[1][ks] = kZero4;
            if (nt < kNT) {
                if constexpr (P % 32 == 0) {   // 16x16x32: p = 32 k + 8 lg + e
#pragma unroll
                    for (int k = 0; k < P / 32; k++) {
                        const float *hp = Hf + (16 * nt + li) * SM::kPH + 32 * k + 8 * lg;
                        s16x4 h0, m0, l0, h1, m1, l1;
                        split4x3(*reinterpret_cast<const f32x4 *>(hp), h0, m0, l0);
                        split4x3(*reinterpret_cast<const f32x4 *>(hp + 4), h1, m1, l1);
                        const bf16x8_t hv = cat8(h0, h1), mv = cat8(m0, m1), lv = cat8(l0, l1);
#pragma unroll
                        for (int jj = 0; jj < 2; jj++) {
                            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(Xs + (16 * kT[jj] + li) * SM::kPX + 32 * k + 8 * lg);
                            dba[jj][ks] = mfma32(a, hv, dba[jj][ks]);
                            dba[jj][ks] = mfma32(a, lv, dba[jj][ks]);
                            dba[jj][ks] = mfma32(a, mv, dba[jj][ks]);
                        }
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < kCT; kk++) {
                        s16x4 hv, mv, lv;
                        split4x3(*reinterpret_cast<const f32x4 *>(Hf + (16 * nt + li) * SM::kPH + 16 * kk + 4 * lg),
                                 hv, mv, lv);
#pragma unroll
                        for (int jj = 0; jj < 2; jj++) {
                            const s16x4 a = *reinterpret_cast<const s16x4 *>(Xs + (16 * kT[jj] + li) * SM::kPX + 16 * kk + 4 * lg);
                            dba[jj][ks] = mfma16(a, hv, dba[jj][ks]);
                            dba[jj][ks] = mfma16(a, lv, dba[jj][ks]);
                            dba[jj][ks] = mfma16(a, mv, dba[jj][ks]);
                        }
                    }
                }
            }
        }
        float qacc[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            const int s0 = 16 * kT[jj] + 4 * lg;
            const f32x4 dv = *reinterpret_cast<const f32x4 *>(dts + s0);
            const f32x4 wb = *reinterpret_cast<const f32x4 *>(wbs + s0);
            if (has_dx) {
#pragma unroll
                for (int r = 0; r < 4; r++)
                    dxa[jj][r] = dv[r] * wb[r] * dxa[jj][r] +
                                 dskip * bf16_to_f32(Ys[(s0 + r) * SM::kPX + 16 * sg + li]);
            }
#pragma unroll
            for (int r = 0; r < 4; r++) qacc[jj][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < kNS; ks++) {
                const int nt = sg + 4 * ks;
                if (nt < kNT) {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        qacc[jj][r] += bf16_to_f32(Bs[(s0 + r) * SM::kPB + 16 * nt + li]) * dba[jj][ks][r];
                        dba[jj][ks][r] *= dv[r] * wb[r];
                    }
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            const float tot = sum16x4(qacc[jj], li);
            if ((li & 3) == 0) Qa[wv * kQ + 16 * kT[jj] + 4 * lg + (li >> 2)] = tot;
        }

        // ---- (t, s) tile pairs with the s tile in kT, one at a time: G and M
        // give W = G L dt_s and dGm = M L dt_s, which enter dx += W^T dy and
        // dB += dGm^T C as A operands.  Lane: t = 16 i + 4 lg + r, s = 16 j + li.
        // The per-step sums below are f64: the gradient w.r.t. a_s is their
        // suffix sum, in which the row and column sums largely cancel.  The
        // four wavefronts of a class hold the same tiles; wavefront sg adds
        // the rows t = 16 i + 4 lg + sg.
        double colg[2] = {0.0, 0.0};   // sum over this lane's row of G L M, s = 16 kT[jj] + li
        double rowv[4] = {0.0, 0.0, 0.0, 0.0};   // sum_s G L M dt_s, row 16 i + 4 lg + sg
#pragma unroll
        for (int pp = 0; pp < 5; pp++) {
            const int i = kPi[pp], j = kPj[pp], jj = j == kT[0] ? 0 : 1;
            f32x4 gacc = kZero4;
#pragma unroll
            for (int k = 0; k < N / 32; k++) {
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(Cs + (16 * i + li) * SM::kPB + 32 * k + 8 * lg);
                const bf16x8_t bb = *reinterpret_cast<const bf16x8_t *>(Bs + (16 * j + li) * SM::kPB + 32 * k + 8 * lg);
                gacc = mfma32(a, bb, gacc);
            }
            const f32x4 macc = rows_dot(Ys, 16 * i, Xs, 16 * j, li, lg);   // M = dy x^T
            const int s = 16 * j + li;
            const float cs = cum[s], csl = cumlo[s], dsv = dts[s];
            const f32x4 ct = *reinterpret_cast<const f32x4 *>(cum + 16 * i + 4 * lg);
            const f32x4 ctl = *reinterpret_cast<const f32x4 *>(cumlo + 16 * i + 4 * lg);
            f32x4 w4, d4;
            float glr[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float e = exp2_hw((ct[r] - cs) + (ctl[r] - csl));
                if (i == j) e = (4 * lg + r >= li) ? e : 0.0f;
                const float gl = gacc[r] * e;
                w4[r] = gl * dsv;
                d4[r] = macc[r] * e * dsv;
                const float glm = gl * macc[r];
                glr[r] = glm;
                if (i == j) dd += (4 * lg + r == li) ? macc[r] : 0.0f;
            }
            {
                // S = G L M dt_s enters a row sum here and, as dt_t times
                // the column sum, the row's own v: exact f64 products, so
                // that the two cancel as they do in exact arithmetic
                const double gs = pick4(glr, sg);
                colg[jj] += gs;
                rowv[i] += sum16d(gs * static_cast<double>(dsv));
            }
            s16x4 wh, wl, mh, ml;
            split4(w4, wh, wl);
            split4(d4, mh, ml);
            if (has_dx) {
                const s16x4 bop = *reinterpret_cast<const s16x4 *>(YT + (16 * sg + li) * SM::kPT + 16 * i + 4 * lg);
                dxa[jj] = mfma16(wh, bop, dxa[jj]);
                dxa[jj] = mfma16(wl, bop, dxa[jj]);
            }
#pragma unroll
            for (int ks = 0; ks < kNS; ks++) {
                const int nt = sg + 4 * ks;
                if (nt < kNT) {
                    const s16x4 bop = *reinterpret_cast<const s16x4 *>(CT + (16 * nt + li) * SM::kPT + 16 * i + 4 * lg);
                    dba[jj][ks] = mfma16(mh, bop, dba[jj][ks]);
                    dba[jj][ks] = mfma16(ml, bop, dba[jj][ks]);
                }
            }
            // keep the pairs apart: the scheduler would otherwise start all
            // five at once and run out of registers
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            double v = colg[jj];
            v = half_swap_sumd(v, false);
            v = half_swap_sumd(v, true);
            if (lg == 0) Ug[wv * kQ + 16 * kT[jj] + li] = v;
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (li == 0) Vr[wv * kQ + 16 * i + 4 * lg + sg] = rowv[i];
        // dx into the row-staging tile, dB terms to the workspace
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            const int s0 = 16 * kT[jj] + 4 * lg;
            if (has_dx) {
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    const uint32_t d2 = pk_bf16(dxa[jj][2 * k], dxa[jj][2 * k + 1]);
                    DX[(s0 + 2 * k) * SM::kPX + 16 * sg + li] = bf16_t(d2 & 0xffffu);
                    DX[(s0 + 2 * k + 1) * SM::kPX + 16 * sg + li] = bf16_t(d2 >> 16);
                }
            }
#pragma unroll
            for (int ks = 0; ks < kNS; ks++) {
                const int nt = sg + 4 * ks;
                if (nt < kNT)
                    *reinterpret_cast<f32x4 *>(pdB + ((c * 4 + kT[jj]) * kNT + nt) * 256 + lane * 4) = dba[jj][ks];
            }
        }

        __builtin_amdgcn_sched_barrier(0);
        // H_in of this chunk as the B operand of dy H_in:
        // hin[ks][kk][e] = H_in[p = poff(kk) + e][n = 16 (sg + 4 ks) + li]: for
        // 16x16x32 products kk = 2 k, 2 k + 1 hold p = 32 k + 8 lg + 0..7
        auto poff = [&](int kk) {
            return P % 32 == 0 ? 32 * (kk >> 1) + 8 * lg + 4 * (kk & 1) : 16 * kk + 4 * lg;
        };
        f32x4 hin[kNS][kCT];
        {
            const float *hs = hin_g + c * N * P;
#pragma unroll
            for (int ks = 0; ks < kNS; ks++) {
                const int nt = sg + 4 * ks;
#pragma unroll
                for (int kk = 0; kk < kCT; kk++)
                    hin[ks][kk] = nt < kNT ? *reinterpret_cast<const f32x4 *>(hs + (16 * nt + li) * P + poff(kk))
                                           : kZero4;
            }
        }

        __builtin_amdgcn_sched_barrier(0);
        // ---- dC for t tiles kT, state tiles sg + 4 ks (lane: t = 16 i + 4 lg + r,
        // n = 16 nt + li): first exp(cum_t) dy H_in and r_t = exp(cum_t) sum_n C (dy H_in)
        f32x4 dca[2][kNS];
        float racc[2][4];
        float hdot = 0.0f;   // <dH, H_in> over this wavefront's (n, p) (class 0)
#pragma unroll
        for (int ii = 0; ii < 2; ii++)
#pragma unroll
            for (int r = 0; r < 4; r++) racc[ii][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < kNS; ks++) {
            const int nt = sg + 4 * ks;
            s16x4 hh4[kCT], hm4[kCT], hl4[kCT];
#pragma unroll
            for (int kk = 0; kk < kCT; kk++) {
                split4x3(hin[ks][kk], hh4[kk], hm4[kk], hl4[kk]);
                if (HF == 0 && nt < kNT) {
                    const f32x4 dv = *reinterpret_cast<const f32x4 *>(Hf + (16 * nt + li) * SM::kPH + poff(kk));
#pragma unroll
                    for (int e = 0; e < 4; e++) hdot += hin[ks][kk][e] * dv[e];
                }
            }
#pragma unroll
            for (int ii = 0; ii < 2; ii++) {
                const int i = kT[ii];
                dca[ii][ks] = kZero4;
                if (nt < kNT) {
                    f32x4 acc = kZero4;
                    if constexpr (P % 32 == 0) {
#pragma unroll
                        for (int k = 0; k < P / 32; k++) {
                            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(Ys + (16 * i + li) * SM::kPX + 32 * k + 8 * lg);
                            acc = mfma32(a, cat8(hh4[2 * k], hh4[2 * k + 1]), acc);
                            acc = mfma32(a, cat8(hm4[2 * k], hm4[2 * k + 1]), acc);
                            acc = mfma32(a, cat8(hl4[2 * k], hl4[2 * k + 1]), acc);
                        }
                    } else {
#pragma unroll
                        for (int kk = 0; kk < kCT; kk++) {
                            const s16x4 a = *reinterpret_cast<const s16x4 *>(Ys + (16 * i + li) * SM::kPX + 16 * kk + 4 * lg);
                            acc = mfma16(a, hh4[kk], acc);
                            acc = mfma16(a, hm4[kk], acc);
                            acc = mfma16(a, hl4[kk], acc);
                        }
                    }
                    const int t0 = 16 * i + 4 * lg;
                    const f32x4 ec = *reinterpret_cast<const f32x4 *>(ecum + t0);
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        racc[ii][r] += bf16_to_f32(Cs[(t0 + r) * SM::kPB + 16 * nt + li]) * acc[r];
                        acc[r] *= ec[r];
                    }
                    dca[ii][ks] = acc;
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
            const float tot = sum16x4(racc[ii], li);
            if ((li & 3) == 0) Ra[wv * kQ + 16 * kT[ii] + 4 * lg + (li >> 2)] = tot;
        }
        if (HF == 0) {
            hdot = wave_sum(hdot);
            if (lane == 0) Hd[wv] = hdot;
        }
        // then the (s, t) tile pairs with the t tile in kT, one at a time:
        // dGm^T = M^T L dt_s (lane: s = 16 j + 4 lg + r, t = 16 i + li) enters
        // dC += dGm B as the A operand
#pragma unroll
        for (int pp = 0; pp < 5; pp++) {
            const int i = kRi[pp], j = kRj[pp], ii = i == kT[0] ? 0 : 1;
            const f32x4 macc = rows_dot(Xs, 16 * j, Ys, 16 * i, li, lg);   // M^T = x dy^T
            const float ctv = cum[16 * i + li], ctvl = cumlo[16 * i + li];
            const f32x4 cs4 = *reinterpret_cast<const f32x4 *>(cum + 16 * j + 4 * lg);
            const f32x4 cs4l = *reinterpret_cast<const f32x4 *>(cumlo + 16 * j + 4 * lg);
            const f32x4 ds4 = *reinterpret_cast<const f32x4 *>(dts + 16 * j + 4 * lg);
            f32x4 d4;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float e = exp2_hw((ctv - cs4[r]) + (ctvl - cs4l[r]));
                if (i == j) e = (4 * lg + r <= li) ? e : 0.0f;
                d4[r] = macc[r] * e * ds4[r];
            }
            s16x4 th, tl;
            split4(d4, th, tl);
#pragma unroll
            for (int ks = 0; ks < kNS; ks++) {
                const int nt = sg + 4 * ks;
                if (nt < kNT) {
                    const s16x4 bop = *reinterpret_cast<const s16x4 *>(BT + (16 * nt + li) * SM::kPT + 16 * j + 4 * lg);
                    dca[ii][ks] = mfma16(th, bop, dca[ii][ks]);
                    dca[ii][ks] = mfma16(tl, bop, dca[ii][ks]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ii = 0; ii < 2; ii++)
#pragma unroll
            for (int ks = 0; ks < kNS; ks++) {
                const int nt = sg + 4 * ks;
                if (nt < kNT)
                    *reinterpret_cast<f32x4 *>(pdC + ((c * 4 + kT[ii]) * kNT + nt) * 256 + lane * 4) = dca[ii][ks];
            }
    };

    if (nch > 0) {
        load_chunk((nch - 1) * kQ);
        stash_chunk((nch - 1) * kQ);
    }
    publish();
    __syncthreads();
    for (int64_t c = nch - 1; c >= 0; c--) {
        const int64_t c0 = c * kQ;
        if (c > 0) load_chunk(c0 - kQ);
        if (cls) chunk(std::integral_constant<int, 1>{}, c);
        else chunk(std::integral_constant<int, 0>{}, c);
        __syncthreads();
        publish();
        if (wv == 0) {
            // per-step results u, v (before this wavefront stashes the next dt)
            const int s = lane, tt = s >> 4;
            const int cl = (tt == 1 || tt == 2) ? 1 : 0;
            float q = 0.0f, R = 0.0f;
            double ugs = 0.0;
#pragma unroll
            for (int s2 = 0; s2 < 4; s2++) {
                q += Qa[(2 * s2 + cl) * kQ + s];
                R += Ra[(2 * s2 + cl) * kQ + s];
                ugs += Ug[(2 * s2 + cl) * kQ + s];
            }
            // row s was summed by the wavefronts with sg = s % 4, one per class
            const double vrs = Vr[(2 * (s & 3)) * kQ + s] + Vr[(2 * (s & 3) + 1) * kQ + s];
            const double dsv = dts[s];
            q *= wbs[s];
            R *= ecum[s];
            const double u = ugs + q;
            double v = vrs + R - dsv * u;
            const double tq = wave_sumd(dsv * q);
            const float hsum = Hd[0] + Hd[2] + Hd[4] + Hd[6];
            if (s == kQ - 1) v += tq + ecum[kQ - 1] * hsum;
            ug[c * kQ + s] = static_cast<float>(u);
            vg[c * kQ + s] = v;
        }
        // the chunk's dx rows: 16-byte stores, P / 8 lanes per row
        if (tid < kVX) {
            const int t = tid / (P / 8), c8 = tid % (P / 8);
            if (c0 + t < L)
                st_global16(dxg + (c0 + t) * xrow + 8 * c8,
                            *reinterpret_cast<const u32x4 *>(DX + t * SM::kPX + 8 * c8));
        }
        if (c > 0) stash_chunk(c0 - kQ);
        __syncthreads();
    }

    if (p.dh0) {
#pragma unroll
        for (int kk = 0; kk < kDH; kk++) {
            const int k = wv + kWaves * kk;
            if (k < kNT * kCT) {
                const int nt = k / kCT, q = k % kCT;
                *reinterpret_cast<f32x4 *>(p.dh0 + (bh * P + 16 * q + li) * N + 16 * nt + 4 * lg) = dH[kk];
            }
        }
    }
    // dD term of this (batch, head): the two sg == 0 wavefronts' diagonal sums
    if (sg == 0) {
        const float t = wave_sum(dd);
        if (lane == 0) Hd[cls] = t;
    }
    __syncthreads();
    if (tid == 0) ws.dDp[bh] = Hd[0] + Hd[1];
}

// Per (batch, head, chunk), one wavefront: the suffix sums of v give the
// gradient w.r.t. a_s = dt_s A; then ddt (w.r.t. the raw dt) and the
// chunk's dA and ddt_bias terms.
__global__ __launch_bounds__(256) void ssd_bwd_dt_kernel(SsdBwdParams p, BwdWs ws, int64_t nch) {
    const int lane = threadIdx.x & 63;
    const int64_t item = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t H = p.nheads, L = p.seqlen;
    if (item >= p.batch * H * nch) return;   // whole wavefronts
    const int64_t c = item % nch, bh = item / nch, h = bh % H, b = bh / H;
    const int64_t t = c * kQ + lane;
    const bool live = t < L;
    const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
    float raw = 0.0f, dtv = 0.0f;
    if (live) {
        raw = bf16_to_f32(static_cast<const bf16_t *>(p.dt)[(b * L + t) * H + h]) + bias;
        dtv = p.softplus ? softplus_f32(raw) : raw;
    }
    const float u = ws.u[item * kQ + lane];
    double da = ws.v[item * kQ + lane];   // f64: the suffix sums cancel heavily
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_down(da, off, 64);
        if (lane + off < 64) da += o;
    }
    const float post = u + p.A[h] * static_cast<float>(da);
    const float draw = live ? post * (p.softplus ? sigmoid_f32(raw) : 1.0f) : 0.0f;
    if (live) static_cast<bf16_t *>(p.ddt)[(b * L + t) * H + h] = f32_to_bf16(draw);
    const double sa = wave_sumd(static_cast<double>(dtv) * da);
    const float sb = wave_sum(draw);
    if (lane == 0) {
        ws.dAp[item] = sa;
        ws.dbp[item] = sb;
    }
}

// dB (or dC) of one (batch, chunk, group): the per-head terms summed over the
// group's heads in order, then written as bf16 rows.
template <int N>
__global__ __launch_bounds__(256) void ssd_bwd_fold_kernel(SsdBwdParams p, BwdWs ws, int64_t nch) {
    constexpr int kNT = N / 16, kSlots = 4 * kNT * 64;
    __shared__ float tile[kQ][N + 4];
    const int tid = threadIdx.x;
    const int64_t H = p.nheads, G = p.ngroups, L = p.seqlen, hpg = H / G;
    const int which = blockIdx.x & 1;
    const int64_t rest = blockIdx.x >> 1;
    const int64_t g = rest % G, bc = rest / G, c = bc % nch, b = bc / nch;
    const float *src = (which ? ws.pdC : ws.pdB) + ((b * H + g * hpg) * nch + c) * kQ * N;
    const int64_t hstride = nch * kQ * N;
    for (int slot = tid; slot < kSlots; slot += 256) {
        // heads in order; four loads in flight at a time
        const float *sp = src + slot * 4;
        f32x4 acc = kZero4;
        int64_t hh = 0;
        for (; hh + 4 <= hpg; hh += 4) {
            const f32x4 v0 = *reinterpret_cast<const f32x4 *>(sp + hh * hstride);
            const f32x4 v1 = *reinterpret_cast<const f32x4 *>(sp + (hh + 1) * hstride);
            const f32x4 v2 = *reinterpret_cast<const f32x4 *>(sp + (hh + 2) * hstride);
            const f32x4 v3 = *reinterpret_cast<const f32x4 *>(sp + (hh + 3) * hstride);
            acc += v0;
            acc += v1;
            acc += v2;
            acc += v3;
        }
        for (; hh < hpg; hh++) acc += *reinterpret_cast<const f32x4 *>(sp + hh * hstride);
        const int ti = slot >> 6, l = slot & 63;
        const int i = ti / kNT, nt = ti % kNT;
#pragma unroll
        for (int r = 0; r < 4; r++) tile[16 * i + 4 * (l >> 4) + r][16 * nt + (l & 15)] = acc[r];
    }
    __syncthreads();
    bf16_t *dst = static_cast<bf16_t *>(which ? p.dC : p.dB) + ((b * L + c * kQ) * G + g) * N;
    for (int v = tid; v < kQ * N / 8; v += 256) {
        const int t = v / (N / 8), c8 = v % (N / 8);
        if (c * kQ + t < L) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; e++)
                o[e] = pk_bf16(tile[t][8 * c8 + 2 * e], tile[t][8 * c8 + 2 * e + 1]);
            st_global16(dst + t * G * N + 8 * c8, o);
        }
    }
}

// dA, ddt_bias, dD of one head: sums over (batch, chunk) in a fixed order.
__global__ __launch_bounds__(256) void ssd_bwd_param_kernel(SsdBwdParams p, BwdWs ws, int64_t nch) {
    __shared__ double red[3][256];
    const int tid = threadIdx.x;
    const int64_t h = blockIdx.x, H = p.nheads;
    double sa = 0.0, sb = 0.0, sd = 0.0;
    const int64_t items = p.batch * nch;
    for (int64_t k = tid; k < items; k += 256) {
        const int64_t b = k / nch, c = k % nch;
        const int64_t o = (b * H + h) * nch + c;
        sa += ws.dAp[o];
        sb += ws.dbp[o];
    }
    for (int64_t b = tid; b < p.batch; b += 256) sd += ws.dDp[b * H + h];
    red[0][tid] = sa;
    red[1][tid] = sb;
    red[2][tid] = sd;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) {
            red[0][tid] += red[0][tid + w];
            red[1][tid] += red[1][tid + w];
            red[2][tid] += red[2][tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        p.dA[h] = static_cast<float>(red[0][0]);
        if (p.ddt_bias) p.ddt_bias[h] = static_cast<float>(red[1][0]);
        if (p.dD) p.dD[h] = static_cast<float>(red[2][0]);
    }
}

template <int N, int P>
void launch_main(const SsdBwdParams &p, const BwdWs &w, hipStream_t stream) {
    hipLaunchKernelGGL((ss_ssd_bwd_kernel<N, P>), dim3(static_cast<unsigned>(p.batch * p.nheads)),
                       dim3(kThr), 0, stream, p, w);
}

template <int N>
hipError_t launch_main_n(const SsdBwdParams &p, const BwdWs &w, hipStream_t stream) {
    switch (p.headdim) {
        case 16: launch_main<N, 16>(p, w, stream); break;
        case 32: launch_main<N, 32>(p, w, stream); break;
        case 48: launch_main<N, 48>(p, w, stream); break;
        case 64: launch_main<N, 64>(p, w, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipSuccess;
}

template <int N>
void launch_fold(const SsdBwdParams &p, const BwdWs &w, int64_t nch, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(p.batch * nch * p.ngroups * 2));
    hipLaunchKernelGGL(ssd_bwd_fold_kernel<N>, grid, dim3(256), 0, stream, p, w, nch);
}

}  // namespace

size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t ngroups, int64_t dstate) {
    (void)ngroups;
    if (batch <= 0 || nheads <= 0) return 0;
    size_t total = 0;
    carve(nullptr, batch, nheads, (seqlen + kQ - 1) / kQ, headdim, dstate, &total);
    return total;
}

hipError_t launch_ssd_bwd(const SsdBwdParams &p, hipStream_t stream) {
    const int64_t Bt = p.batch, L = p.seqlen, H = p.nheads;
    if (H == 0) return hipSuccess;
    const int64_t nch = (L + kQ - 1) / kQ;
    BwdWs w = carve(p.workspace, Bt, H, nch, p.headdim, p.dstate, nullptr);
    if (p.ckpt) w.states = const_cast<float *>(p.ckpt);   // read only
    hipError_t e = hipSuccess;
    if (Bt > 0) {
        if (nch > 0 && !p.ckpt) {
            SsdParams sp = p;   // the forward's arguments
            sp.out = nullptr;
            sp.last_state = nullptr;
            sp.states = w.states;
            e = launch_ssd_states(sp, stream);
            if (e != hipSuccess) return e;
        }
        switch (p.dstate) {
            case 32: e = launch_main_n<32>(p, w, stream); break;
            case 64: e = launch_main_n<64>(p, w, stream); break;
            case 96: e = launch_main_n<96>(p, w, stream); break;
            case 128: e = launch_main_n<128>(p, w, stream); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
        profile_mark(stream);
        if (nch > 0) {
            const int64_t items = Bt * H * nch;
            hipLaunchKernelGGL(ssd_bwd_dt_kernel, dim3(static_cast<unsigned>((items + 3) / 4)),
                               dim3(256), 0, stream, p, w, nch);
            profile_mark(stream);
            switch (p.dstate) {
                case 32: launch_fold<32>(p, w, nch, stream); break;
                case 64: launch_fold<64>(p, w, nch, stream); break;
                case 96: launch_fold<96>(p, w, nch, stream); break;
                case 128: launch_fold<128>(p, w, nch, stream); break;
                default: return hipErrorInvalidValue;
            }
            profile_mark(stream);
        }
    }
    hipLaunchKernelGGL(ssd_bwd_param_kernel, dim3(static_cast<unsigned>(H)), dim3(256), 0, stream,
                       p, w, nch);
    profile_mark(stream);
    return hipGetLastError();
}

}  // namespace ssk
