// ss_kernels.h -- host-side launchers of the gfx950 selective-scan kernels.
// Called by the C ABI layer (ss_api.cpp) after it has validated every
// argument; the launchers only enqueue work and report launch errors.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssk {

// Kernels keep 16 state lanes per row.  dstate N is cut into slices of 16
// states (grid z = slice): slice k holds states 16k .. 16k + 15, and with
// fewer than 16 left its lanes past N carry zero A, B and C (their state
// stays exactly zero).  Per-state tensors are read and written with stride
// N.  Internal buffers (saved block states, workspace partials) are 16 wide
// per slice.  With more than one slice the scan kernels write each slice's
// per-element sums over its states as f32 partials, and a combine kernel
// adds the slices in ascending order together with the per-element terms
// (D u, the gate, their gradients).
constexpr int kMaxState = 256;

__host__ __device__ inline int state_slices(int nstate) { return (nstate + 15) / 16; }

// Up to this many slices the forward runs a row's slices in the same lane
// (their output terms added in registers before the sum over the row's
// lanes): no per-slice partials and no combine kernel.
constexpr int kMaxLaneSlices = 4;

struct ScanParams {
    int64_t batch, dim, seqlen;
    int nstate;   // dstate, 1..kMaxState
    const void *u, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    const float *bias;
    int softplus;
    const float *h0;
};

// What the forward saves for the backward (one f32 buffer, ss_ckpt_size()
// bytes): the state entering every 16-step block, (slice, batch, dim,
// ceil(L / 16), 16), then -- up to kMaxLaneSlices slices (where the forward
// forms the whole output in the lane), at the next 256-byte boundary -- the
// pre-gate output (batch, dim, L), written when z is given (the backward's
// dz reads it; above that the backward adds dz up from per-slice partials).
constexpr int kCkptSpacing = 16;

// block states of one slice, in floats
__host__ __device__ inline size_t ckpt_state_floats(int64_t batch, int64_t dim, int64_t seqlen) {
    return size_t(batch) * size_t(dim) * size_t((seqlen + kCkptSpacing - 1) / kCkptSpacing) * 16;
}
// where the pre-gate output starts, in floats (up to kMaxLaneSlices slices)
__host__ __device__ inline size_t ckpt_ypre_offset(int64_t batch, int64_t dim, int64_t seqlen,
                                                   int nstate) {
    return (ckpt_state_floats(batch, dim, seqlen) * state_slices(nstate) + 63) / 64 * 64;
}
__host__ __device__ inline bool ckpt_has_ypre(int nstate) {
    return state_slices(nstate) <= kMaxLaneSlices;
}
__host__ __device__ inline size_t ckpt_bytes(int64_t batch, int64_t dim, int64_t seqlen,
                                             int nstate) {
    if (batch <= 0 || dim <= 0 || seqlen <= 0) return 0;
    const int ns = state_slices(nstate);
    if (!ckpt_has_ypre(nstate)) return ckpt_state_floats(batch, dim, seqlen) * ns * sizeof(float);
    return (ckpt_ypre_offset(batch, dim, seqlen, nstate) +
            size_t(batch) * size_t(dim) * size_t(seqlen)) *
           sizeof(float);
}

// Time segments.  A long sequence over few (row, state) lanes leaves most of
// the chip idle, so the scan can cut time into nseg segments of seg_len
// steps (a multiple of 64; the last one takes the rest) that run in
// parallel: a summary pass runs every segment but the last from a zero state
// and records its end state and its total decay exp(A sum delta) -- the
// (decay, input) pair of the segment under the scan's associative operator
// (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) -- and each segment then starts
// from the state those pairs give, combined over the segments before it in
// ascending order.  The number of segments depends on (dim, dstate, seqlen)
// only, so a row's bits never depend on the batch size.  Returns nseg (1 =
// one sequential pass) and sets *seg_len.
int scan_segments(int64_t dim, int nstate, int64_t seqlen, int *seg_len);

// Segment summaries, one buffer of 2 x seg_summ_half floats: per (slice,
// summary k < nseg - 1, batch, dim, 16 states) the segment's end value from
// zero, then -- seg_summ_half floats further on -- its total decay.  The
// forward keeps those of segments 0 .. nseg - 2 (k = segment), the
// backward's adjoint those of segments 1 .. nseg - 1 (k = segment - 1).
__host__ __device__ inline size_t seg_summ_index(int nseg, int64_t batch, int64_t dim, int sl,
                                                 int k, int64_t b, int64_t d, int n) {
    return ((size_t(sl) * (nseg - 1) + k) * batch + b) * dim * 16 + d * 16 + n;
}
__host__ __device__ inline size_t seg_summ_half(int nstate, int nseg, int64_t batch, int64_t dim) {
    return size_t(state_slices(nstate)) * (nseg - 1) * batch * dim * 16;
}

struct FwdParams : ScanParams {
    void *out;
    float *last_state;
    float *ckpt;   // block states, or nullptr
    float *ypre;   // pre-gate output (written when z is given), or nullptr
    float *ypart;  // workspace, several slices: (slice, batch, dim, L) partial sums of C h
    int nseg = 1;          // time segments (scan_segments)
    int seg_len = 0;       // steps per segment
    float *summ = nullptr; // workspace, nseg > 1: per (slice, segment < nseg - 1, batch,
                           // dim, 16) the segment's end state from zero, then its decay
    // Causal convolution in front of the scan (conv_width > 0): u holds the
    // convolution's input x, and the scan's u_t = act(bias + sum_k
    // w[d,k] x_{t-H+k}), H = conv_width - 1, act = SiLU or identity,
    // rounded to the io type as the convolution kernel stores it.  The H
    // inputs before t = 0 come from conv_init (batch, dim, H) or are zero;
    // conv_final (batch, dim, H) receives the last H inputs.
    int conv_width = 0;
    int conv_silu = 0;
    const float *conv_w = nullptr;     // (dim, conv_width)
    const float *conv_b = nullptr;     // (dim) or nullptr
    const float *conv_init = nullptr;
    float *conv_final = nullptr;
};

struct BwdParams : ScanParams {
    const void *dout;
    const float *dlast;
    void *du, *ddelta;
    float *dA;
    void *dB, *dC;
    float *dD;
    void *dz;
    float *dbias;
    float *dh0;
    const float *ckpt;  // block states saved by the forward, or nullptr
    const float *ypre;  // pre-gate output saved by the forward with ckpt, or nullptr
    void *workspace;
    int tight_ws;       // workspace sized for this call (bwd_noalloc_bytes), not ss_bwd's
    // The causal convolution fused in front of the scan (conv_width > 0, one
    // 16-state slice): u holds the convolution's input x and is recomputed
    // as the forward formed it; du is not written -- dx (io type, like x),
    // dconv_w (dim, width), dconv_b (dim, or nullptr) and dconv_init
    // (batch, dim, width - 1, or nullptr) receive the convolution's
    // gradients.
    int conv_width = 0;
    int conv_silu = 0;
    const float *conv_w = nullptr;
    const float *conv_b = nullptr;
    const float *conv_init = nullptr;
    void *dx = nullptr;
    float *dconv_w = nullptr;
    float *dconv_b = nullptr;
    float *dconv_init = nullptr;
};

struct DecodeParams {
    int64_t batch, dim;
    int nstate;   // dstate, 1..kMaxState
    float *state;
    const void *u, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    const float *bias;
    int softplus;
    void *out;
};

// Causal depthwise convolution over time (+ SiLU) in front of the scan.
// x, out, dout, dx: (batch, dim, seqlen) io dtype; w, dw: (dim, width) f32;
// bias, dbias: (dim) f32; windows (init, final, dinit, decode state):
// (batch, dim, width - 1) f32.
constexpr int kConvMaxWidth = 4;

struct ConvParams {
    int64_t batch, dim, seqlen;
    int width;  // 1..kConvMaxWidth
    const void *x;
    const float *w, *bias;
    int silu;
    const float *init;  // or nullptr (zeros)
};

struct ConvFwdParams : ConvParams {
    void *out;
    float *final_state;  // or nullptr
};

struct ConvBwdParams : ConvParams {
    const void *dout;
    void *dx;
    float *dw, *dbias, *dinit;  // dbias, dinit may be nullptr
};

struct ConvUpdateParams {
    int64_t batch, dim;
    int width;
    float *state;
    const void *x;
    const float *w, *bias;
    int silu;
    void *out;
};

// Records the next armed profiling event on `stream` (no-op when unarmed).
void profile_mark(hipStream_t stream);

// Compute units of the current device, looked up once per device.
int device_cus();

// Wavefronts per workgroup of the reverse pass (4 channels each).  A
// 12-wavefront (48-channel) group stages B and C once for three times the
// channels and writes a third of the dB / dC partials; it is taken when such
// groups fill every compute unit in no more rounds than 4-wavefront groups
// (3 per compute unit) would.  Else 4.
int scan_waves(int64_t batch, int64_t dim);

size_t fwd_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int nstate);
hipError_t launch_fwd(const FwdParams &p, bool bf16, hipStream_t stream);
// The forward's summary pass alone (p.nseg > 1, p.seg_len and p.summ set):
// the backward runs it before recomputing block states segment by segment.
hipError_t launch_fwd_summaries(const FwdParams &p, bool bf16, hipStream_t stream);
size_t bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int nstate);
hipError_t launch_bwd(const BwdParams &p, bool bf16, hipStream_t stream);

// Allocation-free backward: its workspace is a device array of
// kBwdScratchBytes that the library holds on every device it runs on.
// bwd_noalloc_bytes: the part of it a call needs (its dB / dC partials for
// the call's channel groups, and the block states unless the forward's
// saved record is passed); bwd_scratch: the array's address on the current
// device (looked up once per device).
constexpr size_t kBwdScratchBytes = size_t(96) << 20;
constexpr int kMaxDevices = 64;
size_t bwd_noalloc_bytes(const BwdParams &p, bool bf16);
hipError_t bwd_scratch(void **ptr);
hipError_t launch_state_update(const DecodeParams &p, bool bf16, hipStream_t stream);

// Mamba-2 SSD forward: scalar A per head, state headdim x dstate per head.
// x, out: (batch, L, nheads, headdim) bf16; dt: (batch, L, nheads) bf16;
// B, C: (batch, L, ngroups, dstate) bf16; A, D, dt_bias: (nheads) f32;
// h0, last_state: (batch, nheads, headdim, dstate) f32.
struct SsdParams {
    int64_t batch, seqlen, nheads, ngroups;
    int headdim, dstate;
    const void *x, *dt;
    const float *A;
    const void *B, *C;
    const float *D, *dt_bias;
    int softplus;
    const float *h0;
    void *out;
    float *last_state;
    // states pass only: H_in of every chunk of 64 steps, (batch, head,
    // chunk, dstate, headdim) f32
    float *states;
};
hipError_t launch_ssd_fwd(const SsdParams &p, hipStream_t stream);
hipError_t launch_ssd_states(const SsdParams &p, hipStream_t stream);
// Bytes of the chunk states ss_ssd_fwd can save for ss_ssd_bwd.
size_t ssd_ckpt_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                      int64_t dstate);

// Mamba-2 SSD backward (through the selective-scan backward).  dout, dx:
// (batch, L, nheads, headdim) bf16; ddt: (batch, L, nheads) bf16; dB, dC:
// (batch, L, ngroups, dstate) bf16; dA, dD, ddt_bias: (nheads) f32; dlast,
// dh0: (batch, nheads, headdim, dstate) f32.
struct SsdBwdParams : SsdParams {
    const void *dout;
    const float *dlast;
    void *dx, *ddt;
    float *dA;
    void *dB, *dC;
    float *dD, *ddt_bias, *dh0;
    const float *ckpt;   // chunk states saved by the forward, or NULL
    void *workspace;
};
size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                               int64_t ngroups, int64_t dstate);
hipError_t launch_ssd_bwd(const SsdBwdParams &p, hipStream_t stream);

// Segments (one wavefront each) a row of the convolution is cut into.
int64_t conv_segments(int64_t seqlen);
hipError_t launch_conv_fwd(const ConvFwdParams &p, bool bf16, hipStream_t stream);
hipError_t launch_conv_bwd(const ConvBwdParams &p, bool bf16, hipStream_t stream);
hipError_t launch_conv_update(const ConvUpdateParams &p, bool bf16, hipStream_t stream);

}  // namespace ssk
