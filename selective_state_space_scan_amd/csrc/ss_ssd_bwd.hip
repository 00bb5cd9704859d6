// ss_ssd_bwd.hip -- Mamba-2 SSD backward through the selective-scan backward.
//
// With one group, the SSD recurrence of a head (a headdim x d_state state,
// scalar A, shared dt, B and C) is exactly the selective scan of the
// state-spaces/mamba README ("Usage / Selective SSM") over headdim
// channels with tied parameters: channel (h, p) has u = x[.., h, p],
// delta = dt[.., h], A[(h, p), n] = A[h], D = D[h], and B, C those of the
// group.  The backward therefore runs the selective-scan backward kernels
// (ss_bwd.hip, f32 inside) on the SSD tensors laid out as its
// (channel, time) rows, and sums the tied gradients back per head:
//   dx = du,  ddt[t, h] = sum_p ddelta[(h, p), t],
//   dA[h] = sum_{p,n} dA[(h, p), n],  dD[h] = sum_p dD,  ddt_bias[h] = sum_p.
// dB, dC, dh0 come out directly (h0 / dh0 have the same layout in both).
//
// This is exact but not the chunked (matrix-core) form: it moves each
// element between layouts and runs the sequential per-state scan, so it is
// several times slower than the forward.  Several groups run one call per
// (batch entry, group).
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_tiles.h"

namespace ssk {
namespace {

constexpr int kTile = 64;

// dst (nb, cw, L) f32  <-  src (nb, L, ctot) bf16, columns c0 .. c0 + cw - 1
__global__ __launch_bounds__(256) void rows_from_time_major(const bf16_t *src, int64_t ctot,
                                                            int64_t c0, int64_t cw, int64_t L,
                                                            float *dst) {
    __shared__ float tile[kTile][kTile + 1];
    const int64_t b = blockIdx.z;
    const int64_t t0 = int64_t(blockIdx.x) * kTile, k0 = int64_t(blockIdx.y) * kTile;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    // read: consecutive threads take consecutive columns of one time step
    for (int r = ty; r < kTile; r += 4) {
        const int64_t t = t0 + r, c = k0 + tx;
        float v = 0.0f;
        if (t < L && c < cw) v = bf16_to_f32(src[(b * L + t) * ctot + c0 + c]);
        tile[r][tx] = v;
    }
    __syncthreads();
    // write: consecutive threads take consecutive time steps of one column
    for (int r = ty; r < kTile; r += 4) {
        const int64_t c = k0 + r, t = t0 + tx;
        if (t < L && c < cw) dst[(b * cw + c) * L + t] = tile[tx][r];
    }
}

// dst (nb, L, ctot) bf16, columns c0 .. c0 + cw - 1  <-  src (nb, cw, L) f32
__global__ __launch_bounds__(256) void time_major_from_rows(const float *src, int64_t ctot,
                                                            int64_t c0, int64_t cw, int64_t L,
                                                            bf16_t *dst) {
    __shared__ float tile[kTile][kTile + 1];
    const int64_t b = blockIdx.z;
    const int64_t t0 = int64_t(blockIdx.x) * kTile, k0 = int64_t(blockIdx.y) * kTile;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < kTile; r += 4) {
        const int64_t c = k0 + r, t = t0 + tx;
        float v = 0.0f;
        if (t < L && c < cw) v = src[(b * cw + c) * L + t];
        tile[r][tx] = v;
    }
    __syncthreads();
    for (int r = ty; r < kTile; r += 4) {
        const int64_t t = t0 + r, c = k0 + tx;
        if (t < L && c < cw) dst[(b * L + t) * ctot + c0 + c] = f32_to_bf16(tile[tx][r]);
    }
}

// delta rows (nb, nhg * P, L) f32 from dt (nb, L, H) bf16, heads h0 .. h0 + nhg - 1
__global__ __launch_bounds__(256) void delta_rows(const bf16_t *dt, int64_t H, int64_t h0,
                                                  int64_t nhg, int64_t P, int64_t L, int64_t nb,
                                                  float *dst) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = nb * nhg * P * L;
    if (i >= total) return;
    const int64_t t = i % L, rest = i / L;
    const int64_t c = rest % (nhg * P), b = rest / (nhg * P);
    dst[i] = bf16_to_f32(dt[(b * L + t) * H + h0 + c / P]);
}

// ddt (nb, L, H) bf16, heads h0 .. h0 + nhg - 1  <-  sum over p of ddelta rows
__global__ __launch_bounds__(256) void ddt_from_rows(const float *dd, int64_t H, int64_t h0,
                                                     int64_t nhg, int64_t P, int64_t L,
                                                     int64_t nb, bf16_t *ddt) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= nb * nhg * L) return;
    const int64_t t = i % L, rest = i / L;
    const int64_t hh = rest % nhg, b = rest / nhg;
    const float *src = dd + ((b * nhg + hh) * P) * L + t;
    float s = 0.0f;
    for (int64_t pp = 0; pp < P; pp++) s += src[pp * L];
    ddt[(b * L + t) * H + h0 + hh] = f32_to_bf16(s);
}

// the tied per-channel parameters of heads h0 .. h0 + nhg - 1
__global__ __launch_bounds__(256) void expand_params(const float *A, const float *D,
                                                     const float *bias, int64_t h0, int64_t nhg,
                                                     int64_t P, int64_t N, float *As, float *Ds,
                                                     float *bs) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= nhg * P * N) return;
    const int64_t c = i / N, h = h0 + c / P;
    As[i] = A[h];
    if (i % N == 0) {
        if (D) Ds[c] = D[h];
        if (bias) bs[c] = bias[h];
    }
}

// dA[h] (+)= sum_{p,n}, dD[h], ddt_bias[h] (+)= sum_p, in ascending order
__global__ __launch_bounds__(256) void reduce_params(const float *dAs, const float *dDs,
                                                     const float *dbs, int64_t h0, int64_t nhg,
                                                     int64_t P, int64_t N, int accumulate,
                                                     float *dA, float *dD, float *dbias) {
    const int64_t hh = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (hh >= nhg) return;
    float sa = 0.0f, sd = 0.0f, sb = 0.0f;
    for (int64_t pp = 0; pp < P; pp++) {
        const int64_t c = hh * P + pp;
        for (int64_t n = 0; n < N; n++) sa += dAs[c * N + n];
        if (dD) sd += dDs[c];
        if (dbias) sb += dbs[c];
    }
    const int64_t h = h0 + hh;
    dA[h] = accumulate ? dA[h] + sa : sa;
    if (dD) dD[h] = accumulate ? dD[h] + sd : sd;
    if (dbias) dbias[h] = accumulate ? dbias[h] + sb : sb;
}

// Workspace carve-up for calls over nbc batch entries and nhg heads.
struct SsdBwdWs {
    float *u, *delta, *dout, *du, *ddelta, *Bt, *Ct, *dBt, *dCt;
    float *As, *Ds, *bs, *dAs, *dDs, *dbs;
    void *s6;
    size_t s6_bytes;
};

inline size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

SsdBwdWs carve_ssd(void *base, int64_t nbc, int64_t nhg, int64_t P, int64_t N, int64_t L,
                   size_t *total) {
    const int64_t dim = nhg * P;
    char *p = static_cast<char *>(base);
    size_t off = 0;
    auto take = [&](size_t floats) {
        float *r = reinterpret_cast<float *>(p + off);
        off += a256(floats * sizeof(float));
        return r;
    };
    SsdBwdWs w;
    const size_t E = size_t(nbc) * dim * L, bc = size_t(nbc) * N * L;
    w.u = take(E); w.delta = take(E); w.dout = take(E); w.du = take(E); w.ddelta = take(E);
    w.Bt = take(bc); w.Ct = take(bc); w.dBt = take(bc); w.dCt = take(bc);
    w.As = take(size_t(dim) * N); w.Ds = take(dim); w.bs = take(dim);
    w.dAs = take(size_t(dim) * N); w.dDs = take(dim); w.dbs = take(dim);
    w.s6_bytes = bwd_workspace_bytes(nbc, dim, L, int(N));
    w.s6 = p + off;
    off += a256(w.s6_bytes);
    if (total) *total = off;
    return w;
}

dim3 tgrid(int64_t L, int64_t cw, int64_t nb) {
    return dim3(unsigned((L + kTile - 1) / kTile), unsigned((cw + kTile - 1) / kTile), unsigned(nb));
}
dim3 lgrid(int64_t n) { return dim3(unsigned((n + 255) / 256)); }

}  // namespace

size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t ngroups, int64_t dstate) {
    if (batch <= 0 || nheads <= 0 || ngroups <= 0) return 0;
    const int64_t nbc = ngroups == 1 ? batch : 1;
    size_t total = 0;
    carve_ssd(nullptr, nbc, nheads / ngroups, headdim, dstate, seqlen, &total);
    return total;
}

hipError_t launch_ssd_bwd(const SsdBwdParams &p, hipStream_t stream) {
    const int64_t Bt = p.batch, L = p.seqlen, H = p.nheads, G = p.ngroups;
    const int64_t P = p.headdim, N = p.dstate, nhg = H / G, dim = nhg * P;
    if (Bt == 0 || H == 0) return hipSuccess;
    const bool one = G == 1;
    const int64_t nbc = one ? Bt : 1;
    SsdBwdWs w = carve_ssd(p.workspace, nbc, nhg, P, N, L, nullptr);
    const bf16_t *x = static_cast<const bf16_t *>(p.x), *dt = static_cast<const bf16_t *>(p.dt);
    const bf16_t *B = static_cast<const bf16_t *>(p.B), *C = static_cast<const bf16_t *>(p.C);
    const bf16_t *dy = static_cast<const bf16_t *>(p.dout);
    bf16_t *dx = static_cast<bf16_t *>(p.dx), *ddt = static_cast<bf16_t *>(p.ddt);
    bf16_t *dB = static_cast<bf16_t *>(p.dB), *dC = static_cast<bf16_t *>(p.dC);
    const int64_t calls_b = one ? 1 : Bt;
    for (int64_t g = 0; g < G; g++) {
        const int64_t h0 = g * nhg;
        hipLaunchKernelGGL(expand_params, lgrid(dim * N), dim3(256), 0, stream, p.A, p.D,
                           p.dt_bias, h0, nhg, P, N, w.As, w.Ds, w.bs);
        for (int64_t cb = 0; cb < calls_b; cb++) {
            // batch entries cb .. cb + nbc - 1 of group g
            const int64_t xo = cb * L * H * P, bo = cb * L * G * N, dto = cb * L * H;
            const int64_t L_ = L;
            if (L_ > 0) {
                hipLaunchKernelGGL(rows_from_time_major, tgrid(L, dim, nbc), dim3(256), 0, stream,
                                   x + xo, H * P, h0 * P, dim, L, w.u);
                hipLaunchKernelGGL(rows_from_time_major, tgrid(L, dim, nbc), dim3(256), 0, stream,
                                   dy + xo, H * P, h0 * P, dim, L, w.dout);
                hipLaunchKernelGGL(rows_from_time_major, tgrid(L, N, nbc), dim3(256), 0, stream,
                                   B + bo, G * N, g * N, N, L, w.Bt);
                hipLaunchKernelGGL(rows_from_time_major, tgrid(L, N, nbc), dim3(256), 0, stream,
                                   C + bo, G * N, g * N, N, L, w.Ct);
                hipLaunchKernelGGL(delta_rows, lgrid(nbc * dim * L), dim3(256), 0, stream,
                                   dt + dto, H, h0, nhg, P, L, nbc, w.delta);
            }
            const size_t so = size_t(cb * H + h0) * P * N;   // h0 / dlast / dh0 slice
            BwdParams q{};
            q.batch = nbc; q.dim = dim; q.seqlen = L; q.nstate = int(N);
            q.u = w.u; q.delta = w.delta; q.A = w.As; q.B = w.Bt; q.C = w.Ct;
            q.D = p.D ? w.Ds : nullptr; q.z = nullptr;
            q.bias = p.dt_bias ? w.bs : nullptr; q.softplus = p.softplus;
            q.h0 = p.h0 ? p.h0 + so : nullptr;
            q.dout = w.dout; q.dlast = p.dlast ? p.dlast + so : nullptr;
            q.du = w.du; q.ddelta = w.ddelta; q.dA = w.dAs; q.dB = w.dBt; q.dC = w.dCt;
            q.dD = p.D ? w.dDs : nullptr; q.dz = nullptr; q.dbias = p.dt_bias ? w.dbs : nullptr;
            q.dh0 = p.dh0 ? p.dh0 + so : nullptr;
            q.ckpt = nullptr; q.ypre = nullptr; q.workspace = w.s6;
            hipError_t e = launch_bwd(q, false, stream);
            if (e != hipSuccess) return e;
            if (L_ > 0) {
                hipLaunchKernelGGL(time_major_from_rows, tgrid(L, dim, nbc), dim3(256), 0, stream,
                                   w.du, H * P, h0 * P, dim, L, dx + xo);
                hipLaunchKernelGGL(time_major_from_rows, tgrid(L, N, nbc), dim3(256), 0, stream,
                                   w.dBt, G * N, g * N, N, L, dB + bo);
                hipLaunchKernelGGL(time_major_from_rows, tgrid(L, N, nbc), dim3(256), 0, stream,
                                   w.dCt, G * N, g * N, N, L, dC + bo);
                hipLaunchKernelGGL(ddt_from_rows, lgrid(nbc * nhg * L), dim3(256), 0, stream,
                                   w.ddelta, H, h0, nhg, P, L, nbc, ddt + dto);
            }
            hipLaunchKernelGGL(reduce_params, lgrid(nhg), dim3(256), 0, stream, w.dAs,
                               w.dDs, w.dbs, h0, nhg, P, N, int(cb > 0), p.dA,
                               p.D ? p.dD : nullptr, p.dt_bias ? p.ddt_bias : nullptr);
        }
    }
    profile_mark(stream);
    return hipGetLastError();
}

}  // namespace ssk
