// ss_api.cpp -- the C ABI of libss.so (declared in include/ss.h).
//
// Validates every argument on the host before anything is enqueued, keeps a
// thread-local message naming what failed, and hands valid requests to the
// kernel launchers.  Nothing here allocates device memory or synchronizes.
#include <atomic>
#include "ss.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ss_kernels.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t *g_prof = nullptr;
thread_local int g_prof_count = 0;
thread_local int g_prof_used = 0;
thread_local int g_regime = SS_SCAN_AUTO;   // ss_set_scan_regime

ss_status fail(ss_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

ss_status ok() {
    g_err[0] = '\0';
    return SS_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest extents: batch and channel groups are 32-bit grid coordinates,
// and the kernels address a 16-row tile (16 x seqlen elements of up to
// 4 bytes) with 32-bit byte offsets from a scalar base.
constexpr int64_t kMaxBatch = 65535;
constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxSeq = int64_t(1) << 26;

// HIP launches at most 2^32 - 1 work-items along a grid dimension (blocks
// times threads per block).  Every launcher's x extent is checked against it
// here, on the host, so an oversized shape is refused as unsupported before
// anything is enqueued instead of failing at launch.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;

bool grid_fits(int64_t blocks, int64_t threads) {
    return blocks <= kMaxWorkItems / threads;
}

// Blocks of an elementwise pass over n items, v per thread, 256 threads each.
int64_t elementwise_blocks(int64_t n, int64_t v) { return (n / v + 255) / 256; }

// The x extents of the selective-scan launches for one call: the scan
// kernels (16 or 48 channels per block of 256 or 768 threads), the slice
// combine kernels (several 16-state slices), the backward's fold, and
// decode's 4 lanes per row.
ss_status check_scan_grids(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                           bool bwd) {
    if (!grid_fits((dim + 15) / 16, 256) || !grid_fits((dim + 47) / 48, 768))
        return fail(SS_EUNSUPPORTED,
                    "dim %lld: the scan's launch grid would exceed 2^32 work-items",
                    (long long)dim);
    // batch, dim and seqlen are within check_dims' limits, but their product
    // can pass 2^63
    const __int128 E = static_cast<__int128>(batch) * dim * seqlen;
    const int64_t v = seqlen % 4 == 0 ? 4 : 1;
    if (dstate > 16 && E / v > static_cast<__int128>(kMaxWorkItems) - 255)
        return fail(SS_EUNSUPPORTED,
                    "batch * dim * seqlen: the state-slice combine grid would exceed 2^32 "
                    "work-items");
    if (bwd) {
        const int64_t fold = batch * dstate * seqlen / v + dim * dstate + dim;
        if (!grid_fits(elementwise_blocks(fold, 1), 256))
            return fail(SS_EUNSUPPORTED,
                        "batch * dstate * seqlen: the backward's fold grid would exceed 2^32 "
                        "work-items");
    }
    return SS_OK;
}

struct Check {
    ss_status st = SS_OK;
    // first failure wins
    void need(const void *p, const char *name) {
        if (st != SS_OK) return;
        if (!p) st = fail(SS_EINVAL, "%s must not be NULL", name);
        else if (!aligned16(p)) st = fail(SS_EINVAL, "%s must be 16-byte aligned", name);
    }
    void opt(const void *p, const char *name) {
        if (st != SS_OK || !p) return;
        if (!aligned16(p)) st = fail(SS_EINVAL, "%s must be 16-byte aligned", name);
    }
    void pair(const void *grad, const void *input, const char *gname, const char *iname) {
        if (st != SS_OK) return;
        if ((grad == nullptr) != (input == nullptr))
            st = fail(SS_EINVAL, "%s must be given exactly when %s is given", gname, iname);
    }
};

ss_status check_dims(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io,
                     bool scan) {
    if (batch < 0) return fail(SS_EINVAL, "batch must be >= 0 (got %lld)", (long long)batch);
    if (dim < 0) return fail(SS_EINVAL, "dim must be >= 0 (got %lld)", (long long)dim);
    if (scan && seqlen < 0)
        return fail(SS_EINVAL, "seqlen must be >= 0 (got %lld)", (long long)seqlen);
    if (dstate <= 0) return fail(SS_EINVAL, "dstate must be > 0 (got %lld)", (long long)dstate);
    if (io != SS_F32 && io != SS_BF16)
        return fail(SS_EINVAL, "io_dtype must be SS_F32 (0) or SS_BF16 (1) (got %d)", io);
    if (dstate > ssk::kMaxState)
        return fail(SS_EUNSUPPORTED, "dstate %lld is not supported (this build handles 1..%d)",
                    (long long)dstate, ssk::kMaxState);
    if (scan && batch > kMaxBatch)
        return fail(SS_EUNSUPPORTED, "batch %lld exceeds %lld", (long long)batch,
                    (long long)kMaxBatch);
    if (dim > kMaxDim)
        return fail(SS_EUNSUPPORTED, "dim %lld exceeds %lld", (long long)dim, (long long)kMaxDim);
    if (scan && seqlen > kMaxSeq)
        return fail(SS_EUNSUPPORTED, "seqlen %lld exceeds %lld", (long long)seqlen,
                    (long long)kMaxSeq);
    if (!scan && static_cast<__int128>(batch) * dim > (static_cast<__int128>(1) << 37))
        return fail(SS_EUNSUPPORTED, "batch * dim too large");
    return SS_OK;
}

ss_status device_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(SS_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

namespace ssk {
void profile_mark(hipStream_t stream) {
    if (g_prof && g_prof_used < g_prof_count) (void)hipEventRecord(g_prof[g_prof_used++], stream);
}

int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int scan_segments(int64_t dim, int nstate, int64_t seqlen, int *seg_len) {
    // Wavefronts one batch entry gives the sequential scan: 4 rows of 16
    // states each.  With fewer than 3072 (3 per SIMD of the 256-CU chip) and
    // a long sequence, cut time into segments of at least 1024 steps until
    // one batch entry gives about 6144 (measured at 1536 channels x 16384
    // steps: 8 segments 253 us, 16 segments 231 us).  Short sequences
    // (< 8192 steps) keep one segment: the summary pass would cost more than
    // it gives back at large batches, and the rule cannot look at the batch
    // (a row's bits must not depend on it).  The segmented regime, which a
    // caller asks for when it knows its calls have few rows (a batch-1
    // prefill), takes segments from 1024 steps on, of at least 512 steps
    // (measured at 1 x 1536 x 2048 bf16: forward 75 -> 50 us, step 297 ->
    // 176 us; at 8 x 1536 x 2048 the same segments cost 30%).
    const int64_t waves = (dim + 3) / 4 * state_slices(nstate);
    *seg_len = int(seqlen);
    const bool segmented = g_regime == SS_SCAN_SEGMENTED;
    if (g_regime == SS_SCAN_SEQUENTIAL || waves <= 0 || waves >= 3072) return 1;
    if (seqlen < (segmented ? 1024 : 8192)) return 1;
    const int64_t min_len = segmented ? 512 : 1024;
    int64_t nseg = (6144 + waves - 1) / waves;
    if (nseg > seqlen / min_len) nseg = seqlen / min_len;
    if (nseg > 64) nseg = 64;
    if (nseg < 2) return 1;
    const int64_t len = ((seqlen + nseg - 1) / nseg + 63) / 64 * 64;
    *seg_len = int(len);
    return int((seqlen + len - 1) / len);
}

int scan_waves(int64_t batch, int64_t dim) {
    const int64_t cus = device_cus();
    const int64_t wg4 = batch * ((dim + 15) / 16), wg12 = batch * ((dim + 47) / 48);
    const int64_t rounds4 = (wg4 + 3 * cus - 1) / (3 * cus), rounds12 = (wg12 + cus - 1) / cus;
    return (wg12 >= cus && rounds12 <= rounds4) ? 12 : 4;
}
}  // namespace ssk

extern "C" {

ss_status ss_profile_events(void **events, int count) {
    if (events && count < 0) return fail(SS_EINVAL, "count must be >= 0");
    g_prof = events ? reinterpret_cast<hipEvent_t *>(events) : nullptr;
    g_prof_count = events ? count : 0;
    g_prof_used = 0;
    return ok();
}

int ss_profile_events_used(void) { return g_prof_used; }


int ss_abi_version(void) { return SS_ABI_VERSION; }

ss_status ss_set_scan_regime(int regime) {
    if (regime != SS_SCAN_AUTO && regime != SS_SCAN_SEQUENTIAL && regime != SS_SCAN_SEGMENTED)
        return fail(SS_EINVAL, "unknown scan regime %d", regime);
    g_regime = regime;
    return ok();
}

int ss_scan_regime(void) { return g_regime; }

const char *ss_last_error(void) { return g_err; }

size_t ss_fwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
    if (check_dims(batch, dim, dstate, seqlen, SS_F32, true) != SS_OK) return 0;
    return ssk::fwd_workspace_bytes(batch, dim, seqlen, int(dstate));
}

}  // extern "C"

namespace {

// The causal convolution in front of the scan (ss_fwd_conv), already
// validated by the caller.
struct ConvArgs {
    int width, silu;
    const float *w, *b, *init;
    float *final_state;
};

ss_status fwd_impl(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                   const void *u, const void *delta, const float *A, const void *B, const void *C,
                   const float *D, const void *z, const float *delta_bias, int delta_softplus,
                   const float *h0, void *out, float *last_state, float *ckpt, void *workspace,
                   size_t workspace_bytes, void *stream, const ConvArgs *conv) {
    const char *uname = conv ? "x" : "u";
    ss_status st = check_dims(batch, dim, dstate, seqlen, io_dtype, true);
    if (st != SS_OK) return st;
    st = check_scan_grids(batch, dim, dstate, seqlen, false);
    if (st != SS_OK) return st;
    const bool has_rows = batch > 0 && dim > 0;
    Check c;
    if (has_rows && seqlen > 0) {
        c.need(u, uname);
        c.need(delta, "delta");
        c.need(B, "B");
        c.need(C, "C");
        c.need(out, "out");
    } else {
        c.opt(u, uname); c.opt(delta, "delta"); c.opt(B, "B"); c.opt(C, "C"); c.opt(out, "out");
    }
    if (dim > 0) c.need(A, "A"); else c.opt(A, "A");
    c.opt(D, "D");
    c.opt(z, "z");
    c.opt(delta_bias, "delta_bias");
    c.opt(h0, "h0");
    c.opt(last_state, "last_state");
    c.opt(ckpt, "ckpt");
    if (c.st != SS_OK) return c.st;
    if (h0 && last_state && h0 == last_state)
        return fail(SS_EINVAL, "last_state must not alias h0");
    const size_t need = ssk::fwd_workspace_bytes(batch, dim, seqlen, int(dstate));
    if (need > 0) {
        if (!workspace) return fail(SS_EINVAL, "workspace must not be NULL (%zu bytes needed)", need);
        if (!aligned16(workspace)) return fail(SS_EINVAL, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return fail(SS_EINVAL, "workspace_bytes %zu is smaller than the %zu bytes needed",
                        workspace_bytes, need);
    }
    ssk::FwdParams p{};
    p.batch = batch; p.dim = dim; p.seqlen = seqlen; p.nstate = int(dstate);
    p.u = u; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z;
    p.bias = delta_bias; p.softplus = delta_softplus != 0; p.h0 = h0;
    p.out = out; p.last_state = last_state; p.ckpt = ckpt;
    p.ypre = (ckpt && ssk::ckpt_has_ypre(int(dstate)))
                 ? ckpt + ssk::ckpt_ypre_offset(batch, dim, seqlen, int(dstate)) : nullptr;
    p.ypart = static_cast<float *>(workspace);
    if (conv) {
        p.conv_width = conv->width;
        p.conv_silu = conv->silu;
        p.conv_w = conv->w;
        p.conv_b = conv->b;
        p.conv_init = conv->init;
        p.conv_final = conv->final_state;
    }
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(ssk::launch_fwd(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
                         conv ? "ss_fwd_conv launch" : "ss_fwd launch");
}

}  // namespace

extern "C" {

ss_status ss_fwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int delta_softplus,
                 const float *h0, void *out, float *last_state, float *ckpt, void *workspace,
                 size_t workspace_bytes, void *stream) {
    return fwd_impl(batch, dim, dstate, seqlen, io_dtype, u, delta, A, B, C, D, z, delta_bias,
                    delta_softplus, h0, out, last_state, ckpt, workspace, workspace_bytes, stream,
                    nullptr);
}

size_t ss_ckpt_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
    if (check_dims(batch, dim, dstate, seqlen, SS_F32, true) != SS_OK) return 0;
    return ssk::ckpt_bytes(batch, dim, seqlen, int(dstate));
}

size_t ss_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                             int io_dtype) {
    if (check_dims(batch, dim, dstate, seqlen, io_dtype, true) != SS_OK) return 0;
    return ssk::bwd_workspace_bytes(batch, dim, seqlen, int(dstate));
}

}  // extern "C"

namespace {

// Validation shared by ss_bwd and ss_bwd_noalloc; fills everything of the
// kernel parameters but the workspace.
ss_status bwd_params(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                     const void *u, const void *delta, const float *A, const void *B,
                     const void *C, const float *D, const void *z, const float *delta_bias,
                     int delta_softplus, const float *h0, const void *dout, const float *dlast,
                     void *du, void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz,
                     float *ddelta_bias, float *dh0, const float *ckpt, ssk::BwdParams *p,
                     bool conv = false) {
    // conv: u is the fused convolution's input x, and du is not an output
    const char *uname = conv ? "x" : "u";
    ss_status st = check_dims(batch, dim, dstate, seqlen, io_dtype, true);
    if (st != SS_OK) return st;
    st = check_scan_grids(batch, dim, dstate, seqlen, true);
    if (st != SS_OK) return st;
    const bool has_rows = batch > 0 && dim > 0;
    const bool has_elems = has_rows && seqlen > 0;
    Check c;
    if (has_elems) {
        c.need(u, uname); c.need(delta, "delta"); c.need(dout, "dout");
        if (!conv) c.need(du, "du");
        c.need(ddelta, "ddelta");
    } else {
        c.opt(u, uname); c.opt(delta, "delta"); c.opt(dout, "dout");
        c.opt(du, "du"); c.opt(ddelta, "ddelta");
    }
    if (batch > 0 && seqlen > 0) {
        c.need(B, "B"); c.need(C, "C"); c.need(dB, "dB"); c.need(dC, "dC");
    } else {
        c.opt(B, "B"); c.opt(C, "C"); c.opt(dB, "dB"); c.opt(dC, "dC");
    }
    if (dim > 0) { c.need(A, "A"); c.need(dA, "dA"); } else { c.opt(A, "A"); c.opt(dA, "dA"); }
    c.opt(D, "D"); c.opt(z, "z"); c.opt(delta_bias, "delta_bias"); c.opt(h0, "h0");
    c.opt(dlast, "dlast"); c.opt(dD, "dD"); c.opt(dz, "dz"); c.opt(ddelta_bias, "ddelta_bias");
    c.opt(dh0, "dh0");
    c.opt(ckpt, "ckpt");
    c.pair(dD, D, "dD", "D");
    c.pair(dz, z, "dz", "z");
    c.pair(ddelta_bias, delta_bias, "ddelta_bias", "delta_bias");
    if (c.st != SS_OK) return c.st;
    *p = ssk::BwdParams{};
    p->batch = batch; p->dim = dim; p->seqlen = seqlen; p->nstate = int(dstate);
    p->u = u; p->delta = delta; p->A = A; p->B = B; p->C = C; p->D = D; p->z = z;
    p->bias = delta_bias; p->softplus = delta_softplus != 0; p->h0 = h0;
    p->dout = dout; p->dlast = dlast; p->du = du; p->ddelta = ddelta; p->dA = dA; p->dB = dB;
    p->dC = dC; p->dD = dD; p->dz = dz; p->dbias = ddelta_bias; p->dh0 = dh0; p->ckpt = ckpt;
    p->ypre = (ckpt && ssk::ckpt_has_ypre(int(dstate)))
                  ? ckpt + ssk::ckpt_ypre_offset(batch, dim, seqlen, int(dstate)) : nullptr;
    return SS_OK;
}

}  // namespace

extern "C" {

ss_status ss_bwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int delta_softplus,
                 const float *h0, const void *dout, const float *dlast, void *du, void *ddelta,
                 float *dA, void *dB, void *dC, float *dD, void *dz, float *ddelta_bias,
                 float *dh0, const float *ckpt, void *workspace, size_t workspace_bytes,
                 void *stream) {
    ssk::BwdParams p;
    ss_status st = bwd_params(batch, dim, dstate, seqlen, io_dtype, u, delta, A, B, C, D, z,
                              delta_bias, delta_softplus, h0, dout, dlast, du, ddelta, dA, dB, dC,
                              dD, dz, ddelta_bias, dh0, ckpt, &p);
    if (st != SS_OK) return st;
    const size_t need = ssk::bwd_workspace_bytes(batch, dim, seqlen, int(dstate));
    if (need > 0) {
        if (!workspace) return fail(SS_EINVAL, "workspace must not be NULL (%zu bytes needed)", need);
        if (!aligned16(workspace)) return fail(SS_EINVAL, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return fail(SS_EINVAL, "workspace_bytes %zu is smaller than the %zu bytes needed",
                        workspace_bytes, need);
    }
    p.workspace = workspace;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(ssk::launch_bwd(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
                         "ss_bwd launch");
}

size_t ss_bwd_noalloc_max_scratch(void) { return ssk::kBwdScratchBytes; }

ss_status ss_bwd_noalloc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                         int io_dtype, const void *u, const void *delta, const float *A,
                         const void *B, const void *C, const float *D, const void *z,
                         const float *delta_bias, int delta_softplus, const float *h0,
                         const void *dout, const float *dlast, void *du, void *ddelta, float *dA,
                         void *dB, void *dC, float *dD, void *dz, float *ddelta_bias, float *dh0,
                         const float *ckpt, void *stream) {
    ssk::BwdParams p;
    ss_status st = bwd_params(batch, dim, dstate, seqlen, io_dtype, u, delta, A, B, C, D, z,
                              delta_bias, delta_softplus, h0, dout, dlast, du, ddelta, dA, dB, dC,
                              dD, dz, ddelta_bias, dh0, ckpt, &p);
    if (st != SS_OK) return st;
    const size_t need = ssk::bwd_noalloc_bytes(p, io_dtype == SS_BF16);
    if (need > ssk::kBwdScratchBytes)
        return fail(SS_EUNSUPPORTED,
                    "this shape needs %zu bytes of scratch, more than the %zu ss_bwd_noalloc holds "
                    "(pass the forward's ckpt, or call ss_bwd with a workspace)",
                    need, ssk::kBwdScratchBytes);
    void *scratch = nullptr;
    if (need > 0) {
        const hipError_t e = ssk::bwd_scratch(&scratch);
        if (e != hipSuccess) return device_status(e, "ss_bwd_noalloc scratch lookup");
    }
    p.workspace = scratch;
    p.tight_ws = 1;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(ssk::launch_bwd(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
                         "ss_bwd_noalloc launch");
}

ss_status ss_state_update(int64_t batch, int64_t dim, int64_t dstate, int io_dtype,
                          float *state, const void *u, const void *delta, const float *A,
                          const void *B, const void *C, const float *D, const void *z,
                          const float *delta_bias, int delta_softplus, void *out,
                          void *stream) {
    ss_status st = check_dims(batch, dim, dstate, 1, io_dtype, false);
    if (st != SS_OK) return st;
    // 4 lanes per (batch, channel) row; grid x = channel blocks of 64 rows,
    // grid y = batch entry (at most 65535)
    if (batch > kMaxBatch || !grid_fits((dim + 63) / 64, 256))
        return fail(SS_EUNSUPPORTED,
                    "batch %lld, dim %lld: the state update's launch grid would exceed 2^32 "
                    "work-items or 65535 batch entries", (long long)batch, (long long)dim);
    Check c;
    if (batch > 0 && dim > 0) {
        c.need(state, "state"); c.need(u, "u"); c.need(delta, "delta"); c.need(A, "A");
        c.need(B, "B"); c.need(C, "C"); c.need(out, "out");
    }
    c.opt(D, "D"); c.opt(z, "z"); c.opt(delta_bias, "delta_bias");
    if (c.st != SS_OK) return c.st;
    ssk::DecodeParams p{};
    p.batch = batch; p.dim = dim; p.nstate = int(dstate); p.state = state; p.u = u; p.delta = delta; p.A = A;
    p.B = B; p.C = C; p.D = D; p.z = z; p.bias = delta_bias; p.softplus = delta_softplus != 0;
    p.out = out;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(
        ssk::launch_state_update(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
        "ss_state_update launch");
}

}  // extern "C"

namespace {

ss_status check_conv_dims(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io) {
    if (batch < 0) return fail(SS_EINVAL, "batch must be >= 0 (got %lld)", (long long)batch);
    if (dim < 0) return fail(SS_EINVAL, "dim must be >= 0 (got %lld)", (long long)dim);
    if (seqlen < 0) return fail(SS_EINVAL, "seqlen must be >= 0 (got %lld)", (long long)seqlen);
    if (width < 1) return fail(SS_EINVAL, "width must be >= 1 (got %lld)", (long long)width);
    if (io != SS_F32 && io != SS_BF16)
        return fail(SS_EINVAL, "io_dtype must be SS_F32 (0) or SS_BF16 (1) (got %d)", io);
    if (width > ssk::kConvMaxWidth)
        return fail(SS_EUNSUPPORTED, "width %lld is not supported (this build handles 1..%d)",
                    (long long)width, ssk::kConvMaxWidth);
    if (seqlen > kMaxSeq)
        return fail(SS_EUNSUPPORTED, "seqlen %lld exceeds %lld", (long long)seqlen,
                    (long long)kMaxSeq);
    if (dim > kMaxDim)
        return fail(SS_EUNSUPPORTED, "dim %lld exceeds %lld", (long long)dim, (long long)kMaxDim);
    // forward: one wavefront per (row, segment) in 256-thread blocks;
    // backward: one 128-thread block per channel; decode: one thread per row
    if (batch > 0 && dim > 0 &&
        (batch > kMaxWorkItems / 64 / dim / ssk::conv_segments(seqlen) ||
         !grid_fits(dim, 128) || !grid_fits((batch * dim + 255) / 256, 256)))
        return fail(SS_EUNSUPPORTED,
                    "batch * dim * segments: the convolution's launch grid would exceed 2^32 "
                    "work-items");
    return SS_OK;
}

ss_status check_ssd_dims(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                         int64_t ngroups, int64_t dstate, int io_dtype) {
    if (batch < 0) return fail(SS_EINVAL, "batch must be >= 0 (got %lld)", (long long)batch);
    if (seqlen < 0) return fail(SS_EINVAL, "seqlen must be >= 0 (got %lld)", (long long)seqlen);
    if (nheads < 0) return fail(SS_EINVAL, "nheads must be >= 0 (got %lld)", (long long)nheads);
    if (ngroups < 1 || (nheads > 0 && nheads % ngroups != 0))
        return fail(SS_EINVAL, "ngroups (%lld) must be >= 1 and divide nheads (%lld)",
                    (long long)ngroups, (long long)nheads);
    if (io_dtype != SS_F32 && io_dtype != SS_BF16)
        return fail(SS_EINVAL, "io_dtype must be SS_F32 (0) or SS_BF16 (1) (got %d)", io_dtype);
    if (io_dtype != SS_BF16)
        return fail(SS_EUNSUPPORTED, "the SSD scan runs on bf16 matrix cores: io_dtype must be SS_BF16");
    if (headdim != 16 && headdim != 32 && headdim != 48 && headdim != 64)
        return fail(SS_EUNSUPPORTED, "headdim %lld is not supported (16, 32, 48 or 64)",
                    (long long)headdim);
    if (dstate != 32 && dstate != 64 && dstate != 96 && dstate != 128)
        return fail(SS_EUNSUPPORTED, "dstate %lld is not supported (32, 64, 96 or 128)",
                    (long long)dstate);
    if (seqlen > kMaxSeq)
        return fail(SS_EUNSUPPORTED, "seqlen %lld exceeds %lld", (long long)seqlen,
                    (long long)kMaxSeq);
    // the forward takes one block of 16 * headdim (up to 1024) threads per
    // (batch, head), the backward's chunk kernel one of 512
    if (batch > kMaxBatch || !grid_fits(batch * nheads, 1024))
        return fail(SS_EUNSUPPORTED,
                    "batch * nheads: the SSD launch grid would exceed 2^32 work-items");
    return SS_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

ss_status ss_conv1d_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io_dtype,
                        const void *x, const float *weight, const float *bias, int silu,
                        const float *init_state, void *out, float *final_state, void *stream) {
    ss_status st = check_conv_dims(batch, dim, seqlen, width, io_dtype);
    if (st != SS_OK) return st;
    Check c;
    if (batch > 0 && dim > 0 && seqlen > 0) { c.need(x, "x"); c.need(out, "out"); }
    else { c.opt(x, "x"); c.opt(out, "out"); }
    if (dim > 0) c.need(weight, "weight"); else c.opt(weight, "weight");
    c.opt(bias, "bias");
    c.opt(init_state, "init_state");
    c.opt(final_state, "final_state");
    if (c.st != SS_OK) return c.st;
    const size_t win = size_t(batch) * size_t(dim) * size_t(width - 1) * sizeof(float);
    if (overlaps(init_state, win, final_state, win))
        return fail(SS_EINVAL, "final_state must not overlap init_state");
    ssk::ConvFwdParams p{};
    p.batch = batch; p.dim = dim; p.seqlen = seqlen; p.width = int(width);
    p.x = x; p.w = weight; p.bias = bias; p.silu = silu != 0; p.init = init_state;
    p.out = out; p.final_state = final_state;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(
        ssk::launch_conv_fwd(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
        "ss_conv1d_fwd launch");
}

ss_status ss_fwd_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                      const void *x, const float *conv_weight, int64_t conv_width,
                      const float *conv_bias, int conv_silu, const float *conv_init,
                      const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, void *out, float *last_state,
                      float *conv_final, float *ckpt, void *workspace, size_t workspace_bytes,
                      void *stream) {
    ss_status st = check_conv_dims(batch, dim, seqlen, conv_width, io_dtype);
    if (st != SS_OK) return st;
    if (dstate > 16 * ssk::kMaxLaneSlices && dstate <= ssk::kMaxState)
        return fail(SS_EUNSUPPORTED,
                    "dstate %lld: the fused convolution runs up to %d states (call "
                    "ss_conv1d_fwd, then ss_fwd)",
                    (long long)dstate, 16 * ssk::kMaxLaneSlices);
    Check c;
    if (dim > 0) c.need(conv_weight, "conv_weight"); else c.opt(conv_weight, "conv_weight");
    c.opt(conv_bias, "conv_bias");
    c.opt(conv_init, "conv_init");
    c.opt(conv_final, "conv_final");
    if (c.st != SS_OK) return c.st;
    const size_t win = size_t(batch) * size_t(dim) * size_t(conv_width - 1) * sizeof(float);
    if (overlaps(conv_init, win, conv_final, win))
        return fail(SS_EINVAL, "conv_final must not overlap conv_init");
    // workgroups read inputs of other workgroups' rows and steps (the
    // convolution's halo), so the output may not overwrite them
    const size_t esz = io_dtype == SS_BF16 ? 2 : 4;
    const size_t ebytes = size_t(batch) * size_t(dim) * size_t(seqlen) * esz;
    if (overlaps(x, ebytes, out, ebytes)) return fail(SS_EINVAL, "out must not overlap x");
    const ConvArgs conv{int(conv_width), conv_silu != 0, conv_weight, conv_bias, conv_init,
                        conv_final};
    return fwd_impl(batch, dim, dstate, seqlen, io_dtype, x, delta, A, B, C, D, z, delta_bias,
                    delta_softplus, h0, out, last_state, ckpt, workspace, workspace_bytes, stream,
                    &conv);
}

ss_status ss_bwd_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                      const void *x, const float *conv_weight, int64_t conv_width,
                      const float *conv_bias, int conv_silu, const float *conv_init,
                      const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, const void *dout, const float *dlast,
                      void *dx, float *dconv_weight, float *dconv_bias, float *dconv_init,
                      void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz,
                      float *ddelta_bias, float *dh0, const float *ckpt, void *workspace,
                      size_t workspace_bytes, void *stream) {
    ss_status st = check_conv_dims(batch, dim, seqlen, conv_width, io_dtype);
    if (st != SS_OK) return st;
    if (dstate > 16 && dstate <= ssk::kMaxState)
        return fail(SS_EUNSUPPORTED,
                    "dstate %lld: the fused convolution's backward runs up to 16 states (call "
                    "ss_bwd, then ss_conv1d_bwd)",
                    (long long)dstate);
    ssk::BwdParams p;
    st = bwd_params(batch, dim, dstate, seqlen, io_dtype, x, delta, A, B, C, D, z, delta_bias,
                    delta_softplus, h0, dout, dlast, nullptr, ddelta, dA, dB, dC, dD, dz,
                    ddelta_bias, dh0, ckpt, &p, true);
    if (st != SS_OK) return st;
    Check c;
    if (batch > 0 && dim > 0 && seqlen > 0) c.need(dx, "dx"); else c.opt(dx, "dx");
    if (dim > 0) { c.need(conv_weight, "conv_weight"); c.need(dconv_weight, "dconv_weight"); }
    else { c.opt(conv_weight, "conv_weight"); c.opt(dconv_weight, "dconv_weight"); }
    c.opt(conv_bias, "conv_bias"); c.opt(dconv_bias, "dconv_bias");
    c.opt(conv_init, "conv_init"); c.opt(dconv_init, "dconv_init");
    c.pair(dconv_bias, conv_bias, "dconv_bias", "conv_bias");
    if (c.st != SS_OK) return c.st;
    // workgroups read inputs of other segments' steps (the convolution's
    // window), so dx may not overwrite x
    const size_t ebytes = size_t(batch) * size_t(dim) * size_t(seqlen) * (io_dtype == SS_BF16 ? 2 : 4);
    if (overlaps(x, ebytes, dx, ebytes)) return fail(SS_EINVAL, "dx must not overlap x");
    const size_t need = ssk::bwd_workspace_bytes(batch, dim, seqlen, int(dstate));
    if (need > 0) {
        if (!workspace) return fail(SS_EINVAL, "workspace must not be NULL (%zu bytes needed)", need);
        if (!aligned16(workspace)) return fail(SS_EINVAL, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return fail(SS_EINVAL, "workspace_bytes %zu is smaller than the %zu bytes needed",
                        workspace_bytes, need);
    }
    p.workspace = workspace;
    p.conv_width = int(conv_width);
    p.conv_silu = conv_silu != 0;
    p.conv_w = conv_weight;
    p.conv_b = conv_bias;
    p.conv_init = conv_init;
    p.dx = dx;
    p.dconv_w = dconv_weight;
    p.dconv_b = dconv_bias;
    p.dconv_init = dconv_init;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(ssk::launch_bwd(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
                         "ss_bwd_conv launch");
}

ss_status ss_conv1d_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io_dtype,
                        const void *x, const float *weight, const float *bias, int silu,
                        const float *init_state, const void *dout, void *dx, float *dweight,
                        float *dbias, float *dinit_state, void *stream) {
    ss_status st = check_conv_dims(batch, dim, seqlen, width, io_dtype);
    if (st != SS_OK) return st;
    Check c;
    if (batch > 0 && dim > 0 && seqlen > 0) {
        c.need(x, "x"); c.need(dout, "dout"); c.need(dx, "dx");
    } else {
        c.opt(x, "x"); c.opt(dout, "dout"); c.opt(dx, "dx");
    }
    if (dim > 0) { c.need(weight, "weight"); c.need(dweight, "dweight"); }
    else { c.opt(weight, "weight"); c.opt(dweight, "dweight"); }
    c.opt(bias, "bias"); c.opt(dbias, "dbias");
    c.opt(init_state, "init_state"); c.opt(dinit_state, "dinit_state");
    c.pair(dbias, bias, "dbias", "bias");
    if (c.st != SS_OK) return c.st;
    ssk::ConvBwdParams p{};
    p.batch = batch; p.dim = dim; p.seqlen = seqlen; p.width = int(width);
    p.x = x; p.w = weight; p.bias = bias; p.silu = silu != 0; p.init = init_state;
    p.dout = dout; p.dx = dx; p.dw = dweight; p.dbias = dbias; p.dinit = dinit_state;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(
        ssk::launch_conv_bwd(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
        "ss_conv1d_bwd launch");
}

ss_status ss_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                     int64_t ngroups, int64_t dstate, int io_dtype, const void *x, const void *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const float *dt_bias, int dt_softplus, const float *h0, void *out,
                     float *last_state, float *ckpt, void *stream) {
    ss_status st0 = check_ssd_dims(batch, seqlen, nheads, headdim, ngroups, dstate, io_dtype);
    if (st0 != SS_OK) return st0;
    Check c;
    if (batch > 0 && nheads > 0 && seqlen > 0) {
        c.need(x, "x"); c.need(B, "B"); c.need(C, "C"); c.need(out, "out");
        if (!dt) return fail(SS_EINVAL, "dt must not be NULL");
    } else {
        c.opt(x, "x"); c.opt(B, "B"); c.opt(C, "C"); c.opt(out, "out");
    }
    // dt is read one 2-byte element at a time
    if (dt && (reinterpret_cast<uintptr_t>(dt) & 1u))
        return fail(SS_EINVAL, "dt must be 2-byte aligned");
    if (nheads > 0) c.need(A, "A"); else c.opt(A, "A");
    c.opt(D, "D"); c.opt(dt_bias, "dt_bias"); c.opt(h0, "h0"); c.opt(last_state, "last_state");
    c.opt(ckpt, "ckpt");
    if (c.st != SS_OK) return c.st;
    const size_t st = size_t(batch) * size_t(nheads) * size_t(headdim) * size_t(dstate) * 4;
    if (overlaps(h0, st, last_state, st))
        return fail(SS_EINVAL, "last_state must not overlap h0");
    const size_t ck = ssk::ssd_ckpt_bytes(batch, seqlen, nheads, headdim, dstate);
    if (overlaps(ckpt, ck, h0, st) || overlaps(ckpt, ck, last_state, st))
        return fail(SS_EINVAL, "ckpt must not overlap h0 or last_state");
    ssk::SsdParams p{};
    p.batch = batch; p.seqlen = seqlen; p.nheads = nheads; p.ngroups = ngroups;
    p.headdim = int(headdim); p.dstate = int(dstate);
    p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.dt_bias = dt_bias;
    p.softplus = dt_softplus != 0; p.h0 = h0; p.out = out; p.last_state = last_state;
    p.states = ckpt;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(ssk::launch_ssd_fwd(p, static_cast<hipStream_t>(stream)),
                         "ss_ssd_fwd launch");
}

size_t ss_ssd_ckpt_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate) {
    if (check_ssd_dims(batch, seqlen, nheads, headdim, 1, dstate, SS_BF16) != SS_OK) return 0;
    return ssk::ssd_ckpt_bytes(batch, seqlen, nheads, headdim, dstate);
}

size_t ss_ssd_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                 int64_t ngroups, int64_t dstate) {
    if (check_ssd_dims(batch, seqlen, nheads, headdim, ngroups, dstate, SS_BF16) != SS_OK) return 0;
    return ssk::ssd_bwd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate);
}

ss_status ss_ssd_bwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                     int64_t ngroups, int64_t dstate, int io_dtype, const void *x, const void *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const float *dt_bias, int dt_softplus, const float *h0, const void *dout,
                     const float *dlast, void *dx, void *ddt, float *dA, void *dB, void *dC,
                     float *dD, float *ddt_bias, float *dh0, const float *ckpt,
                     void *workspace, size_t workspace_bytes, void *stream) {
    ss_status st0 = check_ssd_dims(batch, seqlen, nheads, headdim, ngroups, dstate, io_dtype);
    if (st0 != SS_OK) return st0;
    // the per-chunk kernels: batch * nheads * chunks / 4 blocks of 256
    // threads (dt) and batch * chunks * ngroups * 2 blocks of 256 (fold)
    {
        const int64_t nch = (seqlen + 63) / 64;
        if (!grid_fits((batch * nheads * nch + 3) / 4, 256) ||
            !grid_fits(batch * nch * ngroups * 2, 256))
            return fail(SS_EUNSUPPORTED,
                        "batch * nheads * ceil(seqlen / 64): the SSD backward's launch grids "
                        "would exceed 2^32 work-items");
    }
    Check c;
    if (batch > 0 && nheads > 0 && seqlen > 0) {
        c.need(x, "x"); c.need(B, "B"); c.need(C, "C"); c.need(dout, "dout");
        c.need(dx, "dx"); c.need(dB, "dB"); c.need(dC, "dC");
        if (!dt) return fail(SS_EINVAL, "dt must not be NULL");
        if (!ddt) return fail(SS_EINVAL, "ddt must not be NULL");
    } else {
        c.opt(x, "x"); c.opt(B, "B"); c.opt(C, "C"); c.opt(dout, "dout");
        c.opt(dx, "dx"); c.opt(dB, "dB"); c.opt(dC, "dC");
    }
    if ((dt && (reinterpret_cast<uintptr_t>(dt) & 1u)) ||
        (ddt && (reinterpret_cast<uintptr_t>(ddt) & 1u)))
        return fail(SS_EINVAL, "dt and ddt must be 2-byte aligned");
    if (nheads > 0) { c.need(A, "A"); c.need(dA, "dA"); } else { c.opt(A, "A"); c.opt(dA, "dA"); }
    c.opt(D, "D"); c.opt(dt_bias, "dt_bias"); c.opt(h0, "h0"); c.opt(dlast, "dlast");
    c.opt(dD, "dD"); c.opt(ddt_bias, "ddt_bias"); c.opt(dh0, "dh0"); c.opt(ckpt, "ckpt");
    c.pair(dD, D, "dD", "D");
    c.pair(ddt_bias, dt_bias, "ddt_bias", "dt_bias");
    if (c.st != SS_OK) return c.st;
    const size_t need = ssk::ssd_bwd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate);
    if (need > 0) {
        if (!workspace) return fail(SS_EINVAL, "workspace must not be NULL (%zu bytes needed)", need);
        if (!aligned16(workspace)) return fail(SS_EINVAL, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return fail(SS_EINVAL, "workspace_bytes %zu is smaller than the %zu bytes needed",
                        workspace_bytes, need);
    }
    ssk::SsdBwdParams p{};
    p.batch = batch; p.seqlen = seqlen; p.nheads = nheads; p.ngroups = ngroups;
    p.headdim = int(headdim); p.dstate = int(dstate);
    p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.dt_bias = dt_bias;
    p.softplus = dt_softplus != 0; p.h0 = h0; p.out = nullptr; p.last_state = nullptr;
    p.dout = dout; p.dlast = dlast; p.dx = dx; p.ddt = ddt; p.dA = dA; p.dB = dB; p.dC = dC;
    p.dD = dD; p.ddt_bias = ddt_bias; p.dh0 = dh0; p.workspace = workspace; p.ckpt = ckpt;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(ssk::launch_ssd_bwd(p, static_cast<hipStream_t>(stream)),
                         "ss_ssd_bwd launch");
}

ss_status ss_conv1d_update(int64_t batch, int64_t dim, int64_t width, int io_dtype, float *state,
                           const void *x, const float *weight, const float *bias, int silu,
                           void *out, void *stream) {
    ss_status st = check_conv_dims(batch, dim, 1, width, io_dtype);
    if (st != SS_OK) return st;

    Check c;
    if (batch > 0 && dim > 0) {
        c.need(x, "x"); c.need(weight, "weight"); c.need(out, "out");
        if (width > 1) c.need(state, "state"); else c.opt(state, "state");
    } else {
        c.opt(x, "x"); c.opt(weight, "weight"); c.opt(out, "out"); c.opt(state, "state");
    }
    c.opt(bias, "bias");
    if (c.st != SS_OK) return c.st;
    ssk::ConvUpdateParams p{};
    p.batch = batch; p.dim = dim; p.width = int(width); p.state = state; p.x = x;
    p.w = weight; p.bias = bias; p.silu = silu != 0; p.out = out;
    ssk::profile_mark(static_cast<hipStream_t>(stream));
    return device_status(
        ssk::launch_conv_update(p, io_dtype == SS_BF16, static_cast<hipStream_t>(stream)),
        "ss_conv1d_update launch");
}

}  // extern "C"
