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
//   1. checkpoint: the forward recurrence again, writing the state at the
//      start of every 32-step chunk to the workspace;
//   2. reverse: per workgroup of 16 channels x 16 states (one lane per
//      state entry, as in the forward), chunks are visited last to first.
//      Each chunk re-runs its 32 forward steps from its checkpoint, keeping
//      every decay and state in registers, then walks the steps backward.
//      Sums over the 16 states go through a per-wave LDS transpose; sums
//      over the workgroup's 16 channels (dB, dC) through a workgroup LDS
//      tile, written out as one partial per 16 channels;
//   3. fold: adds the dB/dC partials over channel groups in ascending group
//      order and the dA/dD/dbias partials over the batch in ascending batch
//      order.
// Every sum runs in an order fixed by the shape, with no atomics.
#include "ss_device.h"
#include "ss_kernels.h"

namespace ssk {
namespace {

constexpr int kRows = 16;
constexpr int kT = 32;  // chunk length (checkpoint spacing)
constexpr int kThreads = 256;
constexpr int kPitch = kT + 4;
constexpr int kYBlock = kN * 16 + 16;

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
__device__ __forceinline__ void store_vec(T *__restrict__ p, int64_t t, int64_t L, const T *src) {
    if (t + VEC <= L) {
        if constexpr (VEC * sizeof(T) == 16) {
            *reinterpret_cast<Raw16 *>(p + t) = *reinterpret_cast<const Raw16 *>(src);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; e++) p[t + e] = src[e];
        }
    } else {
        for (int e = 0; e < VEC && t + e < L; e++) p[t + e] = src[e];
    }
}

#define SS_BCAST_CASES(X, OUT, J)                                                        \
    switch (J) {                                                                         \
        case 0: OUT = row_bcast<0>(X); break;   case 1: OUT = row_bcast<1>(X); break;    \
        case 2: OUT = row_bcast<2>(X); break;   case 3: OUT = row_bcast<3>(X); break;    \
        case 4: OUT = row_bcast<4>(X); break;   case 5: OUT = row_bcast<5>(X); break;    \
        case 6: OUT = row_bcast<6>(X); break;   case 7: OUT = row_bcast<7>(X); break;    \
        case 8: OUT = row_bcast<8>(X); break;   case 9: OUT = row_bcast<9>(X); break;    \
        case 10: OUT = row_bcast<10>(X); break; case 11: OUT = row_bcast<11>(X); break;  \
        case 12: OUT = row_bcast<12>(X); break; case 13: OUT = row_bcast<13>(X); break;  \
        case 14: OUT = row_bcast<14>(X); break; default: OUT = row_bcast<15>(X); break;  \
    }

template <int M>
__device__ __forceinline__ float xor_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                     (M << 10) | 0x1f));
}

// Sum over the 16 lanes of a DPP row; pairs are combined commutatively, so
// every lane of the row ends with the same bits.
__device__ __forceinline__ float row_sum16(float v) {
    return xor_add<8>(xor_add<4>(xor_add<2>(xor_add<1>(v))));
}

// Workspace carve-up (all f32, 256-byte aligned pieces).
struct Workspace {
    float *ckpt;     // (batch, dim, nck, 16): state entering each chunk
    float *dBp;      // (batch, groups, 16, L)
    float *dCp;      // (batch, groups, 16, L)
    float *dAp;      // (batch, dim, 16)
    float *dDp;      // (batch, dim)
    float *dbiasp;   // (batch, dim)
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline Workspace carve(void *base, int64_t batch, int64_t dim, int64_t L,
                                           size_t *total) {
    const int64_t nck = (L + kT - 1) / kT;
    const int64_t groups = (dim + kRows - 1) / kRows;
    size_t off = 0;
    Workspace w;
    char *p = static_cast<char *>(base);
    auto take = [&](size_t floats) {
        float *r = reinterpret_cast<float *>(p + off);
        off += align256(floats * sizeof(float));
        return r;
    };
    w.ckpt = take(size_t(batch) * dim * nck * kN);
    w.dBp = take(size_t(batch) * groups * kN * L);
    w.dCp = take(size_t(batch) * groups * kN * L);
    w.dAp = take(size_t(batch) * dim * kN);
    w.dDp = take(size_t(batch) * dim);
    w.dbiasp = take(size_t(batch) * dim);
    if (total) *total = off;
    return w;
}

// ---------------------------------------------------------------------------
// kernel 1: checkpoints
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void ss_bwd_ckpt_kernel(BwdParams p, Workspace ws) {
    constexpr int kVecPerRow = kT / VEC;
    constexpr int kVecPerTile = 16 * kVecPerRow;
    constexpr int kTiles = 3;  // B, u, delta
    constexpr int kSlots = (kTiles * kVecPerTile + kThreads - 1) / kThreads;
    __shared__ float sB[kN][kPitch];
    __shared__ __attribute__((aligned(16))) T sU[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sDl[kRows][kT];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, r = wave * 4 + (lane >> 4);
    const int64_t L = p.seqlen, Dm = p.dim, b = blockIdx.y;
    const int64_t d0 = int64_t(blockIdx.x) * kRows, d = d0 + r;
    const bool row_ok = d < Dm;
    const T *gu = static_cast<const T *>(p.u);
    const T *gdl = static_cast<const T *>(p.delta);
    const T *gB = static_cast<const T *>(p.B);
    const float a2 = row_ok ? p.A[d * kN + n] * kLog2e : 0.0f;
    const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    float h = (row_ok && p.h0) ? p.h0[(b * Dm + d) * kN + n] : 0.0f;
    const int64_t nck = (L + kT - 1) / kT;
    float *ck = ws.ckpt + (b * Dm + (row_ok ? d : 0)) * nck * kN + n;

    T pre[kSlots][VEC];
    auto fetch = [&](int64_t t0) {
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            const int slot = tid + k * kThreads;
            const int tile = slot / kVecPerTile, rem = slot % kVecPerTile;
            const int row = rem / kVecPerRow;
            const int64_t t = t0 + (rem % kVecPerRow) * VEC;
            const T *base = gu;
            bool ok = false;
            if (tile == 0) {
                base = gB + (b * kN + row) * L; ok = true;
            } else if (tile < kTiles && d0 + row < Dm) {
                base = (tile == 1 ? gu : gdl) + (b * Dm + d0 + row) * L; ok = true;
            }
            load_vec<T, VEC>(base, t, L, ok, pre[k]);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            const int slot = tid + k * kThreads;
            const int tile = slot / kVecPerTile, rem = slot % kVecPerTile;
            if (tile >= kTiles) continue;
            const int row = rem / kVecPerRow, col = (rem % kVecPerRow) * VEC;
            if (tile == 0) {
#pragma unroll
                for (int e = 0; e < VEC; e++) sB[row][col + e] = to_f32<T>(pre[k][e]);
            } else {
                T *dst = tile == 1 ? &sU[row][col] : &sDl[row][col];
#pragma unroll
                for (int e = 0; e < VEC; e++) dst[e] = pre[k][e];
            }
        }
    };

    if (nck > 0) { fetch(0); stash(); }
    __syncthreads();
    for (int64_t c = 0; c < nck; c++) {
        const int64_t t0 = c * kT;
        if (row_ok) ck[c * kN] = h;
        if (c + 1 < nck) fetch(t0 + kT);
#pragma unroll
        for (int s = 0; s < kT / 16; s++) {
            const int col = 16 * s + n;
            float dl = to_f32<T>(sDl[r][col]) + bias;
            if (p.softplus) dl = softplus_f32(dl);
            if (t0 + col >= L) dl = 0.0f;
            const float dlu = dl * to_f32<T>(sU[r][col]);
#pragma unroll
            for (int j = 0; j < 16; j++) {
                float dj, duj;
                SS_BCAST_CASES(dl, dj, j)
                SS_BCAST_CASES(dlu, duj, j)
                h = __builtin_fmaf(exp2_hw(dj * a2), h, duj * sB[n][16 * s + j]);
            }
        }
        __syncthreads();
        if (c + 1 < nck) stash();
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// kernel 2: reverse pass
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void ss_bwd_reverse_kernel(BwdParams p, Workspace ws) {
    constexpr int kVecPerRow = kT / VEC;
    constexpr int kVecPerTile = 16 * kVecPerRow;
    constexpr int kTiles = 6;  // B, C, u, delta, z, dout
    constexpr int kSlots = (kTiles * kVecPerTile + kThreads - 1) / kThreads;
    __shared__ float sB[kN][kPitch];
    __shared__ float sC[kN][kPitch];
    __shared__ __attribute__((aligned(16))) T sU[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sDl[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sZ[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sG[kRows][kT];   // dout
    __shared__ __attribute__((aligned(16))) T sDu[kRows][kT];  // outputs
    __shared__ __attribute__((aligned(16))) T sDd[kRows][kT];
    __shared__ __attribute__((aligned(16))) T sDz[kRows][kT];
    // shared by the per-wave state transposes and the workgroup channel sums
    __shared__ __attribute__((aligned(16))) float sR[4 * 2 * 4 * kYBlock];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rw = lane >> 4, n = lane & 15, r = wave * 4 + rw;
    const int64_t L = p.seqlen, Dm = p.dim, b = blockIdx.y;
    const int64_t d0 = int64_t(blockIdx.x) * kRows, d = d0 + r;
    const int64_t group = blockIdx.x, groups = gridDim.x;
    const bool row_ok = d < Dm;
    const bool has_z = p.z != nullptr;
    const T *gu = static_cast<const T *>(p.u);
    const T *gdl = static_cast<const T *>(p.delta);
    const T *gz = static_cast<const T *>(p.z);
    const T *gdo = static_cast<const T *>(p.dout);
    const T *gB = static_cast<const T *>(p.B);
    const T *gC = static_cast<const T *>(p.C);

    const float aval = row_ok ? p.A[d * kN + n] : 0.0f;
    const float a2 = aval * kLog2e;
    const float bias = (row_ok && p.bias) ? p.bias[d] : 0.0f;
    const float dskip = (row_ok && p.D) ? p.D[d] : 0.0f;
    const int64_t nck = (L + kT - 1) / kT;
    const float *ck = ws.ckpt + (b * Dm + (row_ok ? d : 0)) * nck * kN + n;

    float g = (row_ok && p.dlast) ? p.dlast[(b * Dm + d) * kN + n] : 0.0f;
    float dA_acc = 0.0f;   // this lane's state entry
    float dD_acc = 0.0f;   // elements t = 16 s + n of this lane's row
    float dbias_acc = 0.0f;

    T pre[kSlots][VEC];
    auto fetch = [&](int64_t t0) {
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            const int slot = tid + k * kThreads;
            const int tile = slot / kVecPerTile, rem = slot % kVecPerTile;
            const int row = rem / kVecPerRow;
            const int64_t t = t0 + (rem % kVecPerRow) * VEC;
            const T *base = gu;
            bool ok = false;
            if (tile == 0) {
                base = gB + (b * kN + row) * L; ok = true;
            } else if (tile == 1) {
                base = gC + (b * kN + row) * L; ok = true;
            } else if (tile < kTiles && d0 + row < Dm && (tile != 4 || has_z)) {
                const T *g0 = tile == 2 ? gu : tile == 3 ? gdl : tile == 4 ? gz : gdo;
                base = g0 + (b * Dm + d0 + row) * L; ok = true;
            }
            load_vec<T, VEC>(base, t, L, ok, pre[k]);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int k = 0; k < kSlots; k++) {
            const int slot = tid + k * kThreads;
            const int tile = slot / kVecPerTile, rem = slot % kVecPerTile;
            if (tile >= kTiles) continue;
            const int row = rem / kVecPerRow, col = (rem % kVecPerRow) * VEC;
            if (tile < 2) {
                float *dst = tile == 0 ? &sB[row][col] : &sC[row][col];
#pragma unroll
                for (int e = 0; e < VEC; e++) dst[e] = to_f32<T>(pre[k][e]);
            } else {
                T *dst = tile == 2 ? &sU[row][col] : tile == 3 ? &sDl[row][col]
                       : tile == 4 ? &sZ[row][col] : &sG[row][col];
#pragma unroll
                for (int e = 0; e < VEC; e++) dst[e] = pre[k][e];
            }
        }
    };

    if (nck > 0) { fetch((nck - 1) * kT); stash(); }
    __syncthreads();

    float *wbuf = &sR[wave * 2 * 4 * kYBlock];  // this wave's transpose region
    for (int64_t c = nck - 1; c >= 0; c--) {
        const int64_t t0 = c * kT;
        if (c > 0) fetch(t0 - kT);
        const float hstart = row_ok ? ck[c * kN] : 0.0f;

        // per-element values, lane (r, n) owns elements 16 s + n
        float dl[2], dlu[2], uu[2], sgd[2], dy[2];
#pragma unroll
        for (int s = 0; s < 2; s++) {
            const int col = 16 * s + n;
            const float raw = to_f32<T>(sDl[r][col]) + bias;
            float x = raw;
            sgd[s] = 1.0f;
            if (p.softplus) {
                x = softplus_f32(raw);
                sgd[s] = sigmoid_f32(raw);
            }
            if (t0 + col >= L) x = 0.0f;
            uu[s] = to_f32<T>(sU[r][col]);
            dl[s] = x;
            dlu[s] = x * uu[s];
        }

        // forward over the chunk from its checkpoint: decays and states
        float ab[kT], hs[kT];
        float h = hstart;
#pragma unroll
        for (int s = 0; s < 2; s++) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; j++) {
                float dj, duj;
                SS_BCAST_CASES(dl[s], dj, j)
                SS_BCAST_CASES(dlu[s], duj, j)
                const int t = 16 * s + j;
                ab[t] = exp2_hw(dj * a2);
                h = __builtin_fmaf(ab[t], h, duj * sB[n][t]);
                hs[t] = h;
                v[j] = sC[n][t] * h;
            }
            const int col = 16 * s + n;
            const float dout = to_f32<T>(sG[r][col]);
            if (has_z) {
                // pre-gate output of element (r, col): transpose-sum over states
#pragma unroll
                for (int q = 0; q < 4; q++)
                    *reinterpret_cast<float4 *>(&wbuf[rw * kYBlock + n * 16 + 4 * q]) =
                        make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
                __builtin_amdgcn_wave_barrier();
                float part[16];
#pragma unroll
                for (int k = 0; k < 16; k++) part[k] = wbuf[rw * kYBlock + k * 16 + n];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int w = 1; w < 16; w *= 2)
#pragma unroll
                    for (int k = 0; k < 16; k += 2 * w) part[k] += part[k + w];
                const float ypre = part[0] + dskip * uu[s];
                const float zz = to_f32<T>(sZ[r][col]);
                const float sz = sigmoid_f32(zz);
                dy[s] = dout * zz * sz;
                sDz[r][col] = from_f32<T>(dout * ypre * sz * (1.0f + zz * (1.0f - sz)));
            } else {
                dy[s] = dout;
            }
            if (t0 + col < L) dD_acc = __builtin_fmaf(dy[s], uu[s], dD_acc);
        }

        // backward over the chunk, 16 steps at a time
#pragma unroll
        for (int s = 1; s >= 0; s--) {
            float qa[16], qb[16], qdb[16], qdc[16];
#pragma unroll
            for (int j = 15; j >= 0; j--) {
                const int t = 16 * s + j;
                float dyj, dj, duj;
                SS_BCAST_CASES(dy[s], dyj, j)
                SS_BCAST_CASES(dl[s], dj, j)
                SS_BCAST_CASES(dlu[s], duj, j)
                g = __builtin_fmaf(sC[n][t], dyj, g);                 // g_t
                const float hprev = t > 0 ? hs[t - 1] : hstart;
                const float gp = g * (ab[t] * hprev);
                dA_acc = __builtin_fmaf(gp, dj, dA_acc);
                qa[j] = aval * gp;
                qb[j] = g * sB[n][t];
                qdb[j] = g * duj;
                qdc[j] = dyj * hs[t];
                g = ab[t] * g;                                        // carried to t-1
            }
            // sums over the 16 states (per-wave transpose)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                *reinterpret_cast<float4 *>(&wbuf[rw * kYBlock + n * 16 + 4 * q]) =
                    make_float4(qa[4 * q], qa[4 * q + 1], qa[4 * q + 2], qa[4 * q + 3]);
                *reinterpret_cast<float4 *>(&wbuf[4 * kYBlock + rw * kYBlock + n * 16 + 4 * q]) =
                    make_float4(qb[4 * q], qb[4 * q + 1], qb[4 * q + 2], qb[4 * q + 3]);
            }
            __builtin_amdgcn_wave_barrier();
            float pa[16], pb[16];
#pragma unroll
            for (int k = 0; k < 16; k++) {
                pa[k] = wbuf[rw * kYBlock + k * 16 + n];
                pb[k] = wbuf[4 * kYBlock + rw * kYBlock + k * 16 + n];
            }
#pragma unroll
            for (int w = 1; w < 16; w *= 2)
#pragma unroll
                for (int k = 0; k < 16; k += 2 * w) {
                    pa[k] += pa[k + w];
                    pb[k] += pb[k + w];
                }
            {
                const int col = 16 * s + n;
                const float sumA = pa[0], sumB = pb[0];
                const float du = __builtin_fmaf(dl[s], sumB, dskip * dy[s]);
                const float dd = __builtin_fmaf(uu[s], sumB, sumA) * sgd[s];
                sDu[r][col] = from_f32<T>(du);
                sDd[r][col] = from_f32<T>(dd);
                if (t0 + col < L) dbias_acc += dd;
            }
            __syncthreads();  // transposes done: the region becomes the channel-sum tile
            // sums over the workgroup's 16 channels: tile [q][row][state][step]
#pragma unroll
            for (int q = 0; q < 4; q++) {
                *reinterpret_cast<float4 *>(&sR[(0 * 16 + r) * 256 + n * 16 + 4 * q]) =
                    make_float4(qdb[4 * q], qdb[4 * q + 1], qdb[4 * q + 2], qdb[4 * q + 3]);
                *reinterpret_cast<float4 *>(&sR[(1 * 16 + r) * 256 + n * 16 + 4 * q]) =
                    make_float4(qdc[4 * q], qdc[4 * q + 1], qdc[4 * q + 2], qdc[4 * q + 3]);
            }
            __syncthreads();
            {
                const int sn = tid >> 4, sj = tid & 15;  // state, step of this thread's sum
                float accb = 0.0f, accc = 0.0f;
#pragma unroll
                for (int rr = 0; rr < kRows; rr++) {
                    accb += sR[(0 * 16 + rr) * 256 + sn * 16 + sj];
                    accc += sR[(1 * 16 + rr) * 256 + sn * 16 + sj];
                }
                const int64_t t = t0 + 16 * s + sj;
                if (t < L) {
                    const int64_t o = ((b * groups + group) * kN + sn) * L + t;
                    ws.dBp[o] = accb;
                    ws.dCp[o] = accc;
                }
            }
            __syncthreads();
        }

        // store this chunk's du, ddelta, dz
        constexpr int kOutVecs = kRows * kT / VEC;
#pragma unroll
        for (int k = 0; k < (kOutVecs + kThreads - 1) / kThreads; k++) {
            const int slot = tid + k * kThreads;
            if (slot < kOutVecs) {
                const int row = slot / (kT / VEC), col = (slot % (kT / VEC)) * VEC;
                if (d0 + row < Dm) {
                    const int64_t base = (b * Dm + d0 + row) * L;
                    store_vec<T, VEC>(static_cast<T *>(p.du) + base, t0 + col, L, &sDu[row][col]);
                    store_vec<T, VEC>(static_cast<T *>(p.ddelta) + base, t0 + col, L, &sDd[row][col]);
                    if (has_z)
                        store_vec<T, VEC>(static_cast<T *>(p.dz) + base, t0 + col, L, &sDz[row][col]);
                }
            }
        }
        if (c > 0) stash();
        __syncthreads();
    }

    // per-row partials of the parameter gradients
    if (row_ok) ws.dAp[(b * Dm + d) * kN + n] = dA_acc;
    // sum the 16 lanes of the row (commutative butterfly: all lanes agree)
    dD_acc = row_sum16(dD_acc);
    dbias_acc = row_sum16(dbias_acc);
    if (row_ok && n == 0) {
        ws.dDp[b * Dm + d] = dD_acc;
        ws.dbiasp[b * Dm + d] = dbias_acc;
    }
    if (p.dh0 && row_ok) p.dh0[(b * Dm + d) * kN + n] = g;
}

// ---------------------------------------------------------------------------
// kernel 3: fixed-order folds
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void ss_bwd_fold_kernel(BwdParams p, Workspace ws) {
    const int64_t L = p.seqlen, Dm = p.dim, Bt = p.batch;
    const int64_t groups = (Dm + kRows - 1) / kRows;
    const int64_t nbc = Bt * kN * L;      // dB / dC elements
    const int64_t na = Dm * kN;           // dA elements
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < nbc) {
        const int64_t bb = i / (kN * L), rem = i - bb * kN * L;  // rem = n * L + t
        float sb = 0.0f, sc = 0.0f;
        for (int64_t gi = 0; gi < groups; gi++) {
            const int64_t o = (bb * groups + gi) * kN * L + rem;
            sb += ws.dBp[o];
            sc += ws.dCp[o];
        }
        static_cast<T *>(p.dB)[i] = from_f32<T>(sb);
        static_cast<T *>(p.dC)[i] = from_f32<T>(sc);
    } else if (i < nbc + na) {
        const int64_t k = i - nbc;
        float s = 0.0f;
        for (int64_t bb = 0; bb < Bt; bb++) s += ws.dAp[bb * na + k];
        p.dA[k] = s;
    } else if (i < nbc + na + Dm) {
        const int64_t dd = i - nbc - na;
        float sD = 0.0f, sb = 0.0f;
        for (int64_t bb = 0; bb < Bt; bb++) {
            sD += ws.dDp[bb * Dm + dd];
            sb += ws.dbiasp[bb * Dm + dd];
        }
        if (p.dD) p.dD[dd] = sD;
        if (p.dbias) p.dbias[dd] = sb;
    }
}

template <typename T>
hipError_t launch_typed(const BwdParams &p, hipStream_t stream) {
    Workspace ws = carve(p.workspace, p.batch, p.dim, p.seqlen, nullptr);
    if (p.batch > 0 && p.dim > 0) {
        dim3 grid(unsigned((p.dim + kRows - 1) / kRows), unsigned(p.batch));
        constexpr int kVec = 16 / sizeof(T);
        if ((p.seqlen * int64_t(sizeof(T))) % 16 == 0) {
            hipLaunchKernelGGL((ss_bwd_ckpt_kernel<T, kVec>), grid, dim3(kThreads), 0, stream, p, ws);
            hipLaunchKernelGGL((ss_bwd_reverse_kernel<T, kVec>), grid, dim3(kThreads), 0, stream, p, ws);
        } else {
            hipLaunchKernelGGL((ss_bwd_ckpt_kernel<T, 1>), grid, dim3(kThreads), 0, stream, p, ws);
            hipLaunchKernelGGL((ss_bwd_reverse_kernel<T, 1>), grid, dim3(kThreads), 0, stream, p, ws);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t total = p.batch * kN * p.seqlen + p.dim * kN + p.dim;
    if (total > 0) {
        hipLaunchKernelGGL((ss_bwd_fold_kernel<T>), dim3(unsigned((total + 255) / 256)), dim3(256),
                           0, stream, p, ws);
    }
    return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen) {
    size_t total = 0;
    carve(nullptr, batch, dim, seqlen, &total);
    return total;
}

hipError_t launch_bwd(const BwdParams &p, bool bf16, hipStream_t stream) {
    return bf16 ? launch_typed<bf16_t>(p, stream) : launch_typed<float>(p, stream);
}

}  // namespace ssk
