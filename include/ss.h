/*
 * ss.h -- C ABI of the MI355X (gfx950) selective state-space scan library
 * (libss.so).
 *
 * The operation is the selective SSM layer of Mamba -- named by the
 * state-spaces/mamba README, section "Usage", subsection "Selective SSM"
 * (the paper's Section 3, Algorithm 2) -- with the full backward pass
 * through the recurrent state and the single-token step on a carried state
 * (mamba-rs README, sections "Features" and "Quick start (CPU)").  The pages
 * print no formula; this library computes, for every batch entry b, channel
 * d and state index n:
 *
 *   delta_t  = delta_raw_t + delta_bias[d]          (bias optional)
 *   delta_t  = softplus(delta_t)                    (if delta_softplus != 0)
 *   h_t[n]   = exp(delta_t * A[d,n]) * h_{t-1}[n] + delta_t * B[b,n,t] * u_t
 *   y_t      = (sum_n C[b,n,t] * h_t[n] + D[d] * u_t) * silu(z_t)
 *
 * with h_{-1} = h0 (zero when h0 is NULL), silu(z) = z * sigmoid(z) applied
 * only when z is given, and the D term only when D is given.
 *
 * Layouts: row-major and contiguous (no strides).
 *   u, delta, z, out, dout, du, ddelta, dz : (batch, dim, seqlen)   io dtype
 *   B, C, dB, dC                           : (batch, dstate, seqlen) io dtype
 *   A, dA                                  : (dim, dstate)           float
 *   D, delta_bias, dD, ddelta_bias         : (dim)                   float
 *   h0, last_state, dlast, dh0             : (batch, dim, dstate)    float
 *   decode: u, delta, z, out (batch, dim); B, C (batch, dstate);
 *           state (batch, dim, dstate) float, updated in place.
 *
 * Numerics.  Inputs are widened exactly to f32; every step, state and
 * reduction runs in f32 (mamba-rs README, "Features": every kernel
 * accumulates in f32; state-spaces/mamba README, "Troubleshooting /
 * Precision": recurrent parameters kept in f32).  bf16 outputs are rounded
 * to nearest-even once, at the store.  Results are deterministic: the same
 * inputs give the same bits on every call, there are no floating-point
 * atomics, and every reduction runs in an order fixed by (dim, dstate,
 * seqlen) alone -- so a row's forward output and decode step are
 * bit-identical whatever the batch size (the batch-invariance contract of
 * the mamba-rs GEMM-modes page, "What is guaranteed").
 *
 * Ownership and streams.  Every pointer except the host scalars is device
 * memory owned by the caller; the library allocates nothing.  Outputs are
 * overwritten, never accumulated into, and must not alias any input (the
 * decode state is the one in-place operand).  Every call enqueues its
 * kernels on `stream` (a hipStream_t; NULL = the default stream) and
 * returns without synchronizing.
 *
 * Errors.  Failures are reported as values that name what failed, never by
 * a hidden fallback (the error convention of the mamba-rs GEMM-modes page,
 * section "Errors", whose calls return a result carrying a message and
 * whose deterministic mode refuses what it cannot honour).  Arguments are
 * validated on the host before anything is launched; on failure nothing is
 * enqueued, the call returns a non-zero ss_status and ss_last_error()
 * (thread-local) names the argument or the HIP call that failed.  A shape
 * whose launch grid would exceed the HIP limit of 2^32 work-items per
 * dimension is refused with SS_EUNSUPPORTED before any launch.  Launch
 * failures return SS_EDEVICE.
 */
#ifndef SS_H
#define SS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_ABI_VERSION 12

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

typedef enum {
    SS_OK = 0,
    SS_EINVAL = 1,       /* bad argument: null/misaligned pointer, bad size, bad combination */
    SS_EUNSUPPORTED = 2, /* valid request this build does not implement (e.g. dstate > 256) */
    SS_EDEVICE = 3       /* a HIP call or kernel launch failed */
} ss_status;

/* SS_ABI_VERSION of the loaded library: lets a caller refuse a library
 * built for another argument list instead of misreading it (the explicit,
 * erroring boundary of the mamba-rs GEMM-modes page, section "Errors"). */
int ss_abi_version(void);

/* Message of the last failed call on this thread ("" after a success): the
 * named-failure half of the error convention of the mamba-rs GEMM-modes
 * page, section "Errors".  The pointer stays valid until the thread's next
 * call into the library. */
const char *ss_last_error(void);

/*
 * Scan regimes.  The mamba-rs GEMM-modes page, section "What is guaranteed",
 * names a sequential and a parallel scan regime, each giving the same bits
 * run to run; each regime here also gives a row the same bits at every
 * batch size, because its choice depends only on (dim, dstate, seqlen),
 * never on the batch.  The two are separate bit families (the parallel one
 * combines per-segment (decay, end state) pairs; both agree with the
 * oracle to the same tolerance).
 *   SS_SCAN_AUTO (the default): time segments only for sequences of 8192
 *     steps or more whose batch entry gives fewer than 3072 wavefronts
 *     (dim / 4 x ceil(dstate / 16)); every other call sequential.
 *   SS_SCAN_SEQUENTIAL: never time segments.
 *   SS_SCAN_SEGMENTED: time segments of at least 512 steps from 1024 steps
 *     on, for the same narrow calls: the latency regime for calls with few
 *     rows (a batch-1 prefill), which at large batches costs about 30%.
 * ss_set_scan_regime sets the regime of the calling thread for every later
 * ss_fwd, ss_fwd_conv, ss_bwd, ss_bwd_conv, ss_bwd_noalloc call and
 * workspace-size query on it (SS_EINVAL for an unknown value; the setting
 * is unchanged then).  A backward that reads a forward's saved record
 * should run in the forward's regime (in another it is still correct, but
 * in neither bit family).  ss_scan_regime returns the thread's setting.
 */
typedef enum { SS_SCAN_AUTO = 0, SS_SCAN_SEQUENTIAL = 1, SS_SCAN_SEGMENTED = 2 } ss_scan_regime_t;
ss_status ss_set_scan_regime(int regime);
int ss_scan_regime(void);

/*
 * Bytes of what ss_fwd can save for ss_bwd (its "ckpt" buffer), all f32:
 * the state entering every 16-step block, per slice of 16 states,
 * (ceil(dstate / 16), batch, dim, ceil(seqlen / 16), 16) -- 16 entries per
 * slice, the unused ones zero.  With dstate <= 64 it is followed, at the
 * next 256-byte boundary, by the pre-gate output sum_n C h + D u, (batch,
 * dim, seqlen), which is written when z is given (ss_bwd's dz reads it
 * instead of adding up per-slice parts).  0 for empty or unsupported
 * shapes.
 */
size_t ss_ckpt_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen);

/* Bytes of device workspace ss_fwd needs (f32, 0 when none):
 *   - above 64 states, the per-slice partial sums over states,
 *     ceil(dstate / 16) * batch * dim * seqlen floats (up to 64 states the
 *     slices of a row meet in the same lanes and need none);
 *   - for a long sequence over few channels (seqlen >= 8192 and fewer than
 *     3072 wavefronts of 4 channels x 16 states per batch entry), the time
 *     segments' summaries: 2 * ceil(dstate / 16) * (nseg - 1) * batch * dim
 *     * 16 floats, nseg = the number of segments (at most 64), after the
 *     partials at the next 256-byte boundary.
 * Whether the scan is cut into time segments, and into how many, depends on
 * (dim, dstate, seqlen) only: a row's results never depend on the batch
 * size. */
size_t ss_fwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen);

/*
 * Forward scan.  Writes out (batch, dim, seqlen) and, when last_state is
 * non-NULL, the final state h_{seqlen-1} (h0 when seqlen == 0).  When ckpt
 * is non-NULL (ss_ckpt_size() bytes, 16-byte aligned) it also saves the
 * block states (and, for dstate <= 64, the pre-gate output), which a later
 * ss_bwd with the same inputs takes instead of recomputing them (the usual
 * save-for-backward of a training step).
 *   dstate            1..256 (SS_EUNSUPPORTED above; the mamba-rs README,
 *                     "Features", sizes state dimensions up to 256).  Above
 *                     16 the states are cut into 16-state slices: up to 64
 *                     a lane runs one state of each slice of its row and
 *                     adds a step's terms over the slices in ascending
 *                     order before the sum over its row's lanes; above 64
 *                     one pass runs per slice and the slices' sums are
 *                     added in ascending order.
 *   Long sequences over few channels (see ss_fwd_workspace_size) run as
 *   parallel time segments: a first pass gives every segment but the last
 *   its (total decay, end state from zero) pair -- the scan's associative
 *   operator (a1, b1) o (a2, b2) = (a1 a2, a2 b1 + b2) applied to the
 *   segment -- and each segment then starts from the state those pairs give
 *   over the segments before it, combined in ascending order.
 *   workspace         ss_fwd_workspace_size() bytes of caller-owned device
 *                     memory, 16-byte aligned (NULL when that is 0).
 *   io_dtype          SS_F32 or SS_BF16: dtype of u, delta, B, C, z, out.
 *   D, z, delta_bias, h0, last_state may be NULL.
 *   batch, dim, seqlen >= 0; a zero size enqueues nothing but the
 *   last_state copy/zero fill it implies.  seqlen <= 2^26, batch <= 65535,
 *   dim <= 2^30 (SS_EUNSUPPORTED beyond; the same limits hold for ss_bwd).
 *   All pointers 16-byte aligned.
 */
ss_status ss_fwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *B,
                 const void *C, const float *D, const void *z, const float *delta_bias,
                 int delta_softplus, const float *h0, void *out, float *last_state,
                 float *ckpt, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace ss_bwd needs for this shape (0 for empty shapes). */
size_t ss_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                             int io_dtype);

/*
 * Backward (reverse-time BPTT) of the loss
 *     sum(dout * out) + sum(dlast * last_state)
 * with respect to every input of ss_fwd with the same arguments.
 *   dout               (batch, dim, seqlen) io dtype; required.
 *   dlast              (batch, dim, dstate) f32 or NULL (no gradient on last_state).
 *   du, ddelta         required; ddelta is the gradient w.r.t. the raw delta argument.
 *   dA                 required, (dim, dstate); summed over batch and time.
 *   dB, dC             required, (batch, dstate, seqlen); summed over channels.
 *   dD                 NULL iff D is NULL; summed over batch and time.
 *   dz                 NULL iff z is NULL.
 *   ddelta_bias        NULL iff delta_bias is NULL; summed over batch and time.
 *   dh0                optional (may be non-NULL with h0 NULL: gradient at a zero start).
 *   ckpt               what ss_fwd saved for exactly these inputs, or NULL
 *                      (then the block states are recomputed in the workspace).
 *   workspace          device memory of at least ss_bwd_workspace_size() bytes,
 *                      16-byte aligned, owned by the caller, not read before written.
 * Every sum over batch, time or channels runs in a fixed order, with no
 * atomics, so the gradients are bit-reproducible.
 * Above 16 states the reverse pass runs once per 16-state slice, and du and
 * ddelta add up over the slices in ascending order: up to 64 states with z,
 * or at any dstate without z, the slices run one launch after another, each
 * adding its parts to the running sums in the workspace and the last adding
 * the D terms and writing du and ddelta; above 64 states with z they run
 * side by side and a final pass adds their parts (dz included).
 * Long sequences over few channels run as ss_fwd's time segments (the same
 * count, from dim, dstate and seqlen only): the block states segment by
 * segment after the forward's summary pass (when ckpt is NULL), then the
 * reverse pass segment by segment after an adjoint summary pass -- each
 * segment but the first records, from a zero adjoint, the adjoint leaving
 * its first step and its total decay exp(A sum delta), and a segment's
 * entering adjoint combines those of the later segments from the last down.
 * The dA, dD and ddelta_bias sums then run over (batch entry, segment) in
 * ascending order.
 */
ss_status ss_bwd(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                 const void *u, const void *delta, const float *A, const void *B,
                 const void *C, const float *D, const void *z, const float *delta_bias,
                 int delta_softplus, const float *h0, const void *dout, const float *dlast,
                 void *du, void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz,
                 float *ddelta_bias, float *dh0, const float *ckpt, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * ss_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and kernels as ss_bwd (bit-identical
 * results), without the workspace: it uses a file-scope device array of
 * ss_bwd_noalloc_max_scratch() bytes (96 MiB) that the library holds on
 * every GPU it runs on until the process ends.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *   The part a call needs is its dB / dC partials, plus the block states
 *   when ckpt is NULL: about 68 MB at batch 8, dim 1536, seqlen 2048,
 *   dstate 16 with the forward's ckpt.  A larger need returns
 *   SS_EUNSUPPORTED with a message; pass ckpt or call ss_bwd.
 *   Every call on a GPU shares that GPU's array, which keeps the last call's
 *   contents (each word is written before it is read, so nothing needs
 *   clearing): calls that overlap on one GPU -- on different streams or
 *   from several threads -- race and must be serialized by the caller.
 */
size_t ss_bwd_noalloc_max_scratch(void);
ss_status ss_bwd_noalloc(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                         int io_dtype, const void *u, const void *delta, const float *A,
                         const void *B, const void *C, const float *D, const void *z,
                         const float *delta_bias, int delta_softplus, const float *h0,
                         const void *dout, const float *dlast, void *du, void *ddelta, float *dA,
                         void *dB, void *dC, float *dD, void *dz, float *ddelta_bias, float *dh0,
                         const float *ckpt, void *stream);

/*
 * One-token state update (decode): advances `state` (batch, dim, dstate,
 * f32, in place) by one step of the recurrence with the token's u, delta,
 * z (batch, dim) and B, C (batch, dstate), and writes out (batch, dim).
 * Each (b, d) row is computed by its own lanes in one fixed order, so a row
 * gives the same bits whether it is stepped alone or inside any batch.
 *   dstate 1..256; D, z, delta_bias may be NULL.
 */
ss_status ss_state_update(int64_t batch, int64_t dim, int64_t dstate, int io_dtype,
                          float *state, const void *u, const void *delta, const float *A,
                          const void *B, const void *C, const float *D, const void *z,
                          const float *delta_bias, int delta_softplus, void *out,
                          void *stream);

/*
 * Causal depthwise convolution over time, the local convolution of width
 * d_conv (4 in the state-spaces/mamba README, "Usage", Mamba block) that
 * feeds the scan's u, with the window the mamba-rs README ("Quick start
 * (CPU)") keeps in its decode state.  For batch b, channel d, K = width,
 * H = K - 1:
 *
 *   pre_t = bias[d] + sum_{k=0}^{K-1} weight[d,k] * x_{t-H+k}
 *   out_t = silu(pre_t) if silu != 0, else pre_t
 *
 * where x_{-H} .. x_{-1} are init_state[b,d,0..H-1] (zeros when init_state
 * is NULL).  The pages print no formula; this is the plainest reading of a
 * causal per-channel convolution in front of the scan.
 *
 * Layouts (row-major, contiguous):
 *   x, out, dout, dx            : (batch, dim, seqlen)   io dtype
 *   weight, dweight             : (dim, width)           float
 *   bias, dbias                 : (dim)                  float
 *   init_state, final_state,
 *   dinit_state, decode state   : (batch, dim, width-1)  float
 *   decode x, out               : (batch, dim)           io dtype
 * width 1..4 (SS_EUNSUPPORTED above 4); seqlen <= 2^26; all pointers
 * 16-byte aligned.  Every sum runs in f32 in a fixed order; results are
 * bit-reproducible and a row's out / dx do not depend on the batch size.
 */

/*
 * Forward.  Writes out and, when final_state is non-NULL, the last H inputs
 * x_{L-H} .. x_{L-1} (reaching into init_state, or zeros, when seqlen < H),
 * so a following call with init_state = that final_state continues the
 * sequence.  bias, init_state, final_state may be NULL; final_state must
 * not overlap init_state.
 */
ss_status ss_conv1d_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io_dtype,
                        const void *x, const float *weight, const float *bias, int silu,
                        const float *init_state, void *out, float *final_state, void *stream);

/*
 * Backward of sum(dout * out) with respect to x (dx, required), weight
 * (dweight, required; summed over batch and time), bias (dbias, given
 * exactly when bias is) and the initial window (dinit_state, optional; may
 * be given without init_state: the gradient at a zero window).  Needs no
 * workspace: the sums over batch and time stay on chip.
 */
ss_status ss_conv1d_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int io_dtype,
                        const void *x, const float *weight, const float *bias, int silu,
                        const float *init_state, const void *dout, void *dx, float *dweight,
                        float *dbias, float *dinit_state, void *stream);

/*
 * Decode step: out = act(bias + sum_k weight[d,k] * window_k) with window =
 * (state[b,d,0..H-1], x[b,d]); then state drops its oldest entry and takes
 * x (in place).  state may be NULL when width == 1.
 */
ss_status ss_conv1d_update(int64_t batch, int64_t dim, int64_t width, int io_dtype, float *state,
                           const void *x, const float *weight, const float *bias, int silu,
                           void *out, void *stream);

/*
 * The convolution fused into the scan's load stage: ss_fwd with
 *   u = ss_conv1d_fwd(x, conv_weight, conv_bias, conv_silu, conv_init)
 * computed per element inside the scan (the state-spaces/mamba README,
 * "Usage", Mamba block: a d_conv = 4 convolution right in front of the
 * SSM; the mamba-rs README, "Features", lists scan and convolution kernels
 * together).  u never reaches memory.  Each u is rounded to the io dtype
 * exactly as ss_conv1d_fwd stores it, so the outputs, last_state, the
 * saved ckpt and conv_final are the same bits as ss_conv1d_fwd followed by
 * ss_fwd on its output -- a training step can take the backward through
 * ss_bwd (with u from ss_conv1d_fwd and this call's ckpt) and
 * ss_conv1d_bwd.
 *   x                  (batch, dim, seqlen) io dtype: the convolution's input.
 *   conv_weight        (dim, conv_width) f32, required; conv_width 1..4.
 *   conv_bias          (dim) f32 or NULL.
 *   conv_init          (batch, dim, conv_width - 1) f32 or NULL (zeros).
 *   conv_final         (batch, dim, conv_width - 1) f32 or NULL: receives the
 *                      last conv_width - 1 inputs (as ss_conv1d_fwd's
 *                      final_state); must not overlap conv_init.
 *   The scan arguments are ss_fwd's.  dstate 1..64 (SS_EUNSUPPORTED above:
 *   call ss_conv1d_fwd, then ss_fwd).  out must not overlap x (workgroups
 *   read other rows' and steps' inputs for the convolution's window).
 *   Workspace: ss_fwd_workspace_size().
 */
ss_status ss_fwd_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                      const void *x, const float *conv_weight, int64_t conv_width,
                      const float *conv_bias, int conv_silu, const float *conv_init,
                      const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, void *out, float *last_state,
                      float *conv_final, float *ckpt, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * Backward of ss_fwd_conv with the convolution's backward fused into the
 * scan's reverse pass: u is recomputed from x exactly as the forward formed
 * it, and the gradient reaching u goes straight through the convolution
 * (du never reaches memory).  Gradients of the loss
 *     sum(dout * out) + sum(dlast * last_state)
 * with respect to x (dx, required, io dtype), conv_weight (dconv_weight,
 * required, summed over batch and time), conv_bias (dconv_bias, given
 * exactly when conv_bias is), the initial window (dconv_init, optional; may
 * be given without conv_init: the gradient at a zero window), and the
 * scan's other inputs as in ss_bwd.  dstate 1..16 (SS_EUNSUPPORTED above:
 * call ss_bwd, then ss_conv1d_bwd).  ckpt: what ss_fwd_conv saved for
 * these inputs, or NULL.  dx must not overlap x.  Workspace:
 * ss_bwd_workspace_size().  With time segments the input gradients of a
 * segment's last conv_width - 1 steps are completed after the reverse pass
 * from the next segment's first pre-activation gradients, in the order one
 * pass adds them.
 */
ss_status ss_bwd_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, int io_dtype,
                      const void *x, const float *conv_weight, int64_t conv_width,
                      const float *conv_bias, int conv_silu, const float *conv_init,
                      const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias,
                      int delta_softplus, const float *h0, const void *dout, const float *dlast,
                      void *dx, float *dconv_weight, float *dconv_bias, float *dconv_init,
                      void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz,
                      float *ddelta_bias, float *dh0, const float *ckpt, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Mamba-2 SSD forward: the selective scan with a scalar A per head (the SSD
 * module the state-spaces/mamba README names under "Mamba-2"; d_state
 * typically 64 or 128).  The pages print no formula; the reading is, per
 * batch b and head h with a headdim x dstate state H,
 *
 *   dt_t = softplus(dt[b,t,h] + dt_bias[h])    (bias, softplus optional)
 *   H_t  = exp(dt_t A[h]) H_{t-1} + dt_t x_t B_t^T
 *   y_t  = H_t C_t + D[h] x_t
 *
 * with B and C shared by a group of nheads / ngroups consecutive heads and
 * H_{-1} = h0 (zero when NULL).  Computed in chunks of 64 steps on bf16
 * matrix cores with f32 accumulation.  The chunked form needs decays:
 * dt_t A[h] <= 0 (A negative, and dt non-negative, which softplus ensures);
 * a growing state overflows.
 *
 * Layouts (row-major, contiguous; time-major like the mamba-rs Mamba-3
 * scratch buffers):
 *   x, out          : (batch, seqlen, nheads, headdim)   bf16
 *   dt              : (batch, seqlen, nheads)            bf16 (raw, before bias/softplus)
 *   B, C            : (batch, seqlen, ngroups, dstate)   bf16
 *   A, D, dt_bias   : (nheads)                           float
 *   h0, last_state  : (batch, nheads, headdim, dstate)   float
 * io_dtype must be SS_BF16 (SS_EUNSUPPORTED otherwise); headdim 16, 32, 48
 * or 64; dstate 32, 64, 96 or 128; ngroups divides nheads; seqlen <= 2^26;
 * batch <= 65535 and batch * nheads < 2^22 (one workgroup of up to 1024
 * threads per (batch, head); SS_EUNSUPPORTED beyond).
 * D, dt_bias, h0, last_state may be NULL; last_state must not overlap h0.
 * ckpt, when non-NULL (ss_ssd_ckpt_size() bytes, f32), receives the state
 * entering every chunk of 64 steps, which a later ss_ssd_bwd with the same
 * inputs takes instead of recomputing it (save-for-backward); it must not
 * overlap h0 or last_state.
 * Pointers 16-byte aligned, except dt (2-byte aligned suffices).
 * Each (batch, head) is computed by one workgroup in a fixed order, so the
 * results are bit-reproducible and do not depend on the batch size.
 */
ss_status ss_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                     int64_t ngroups, int64_t dstate, int io_dtype, const void *x, const void *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const float *dt_bias, int dt_softplus, const float *h0, void *out,
                     float *last_state, float *ckpt, void *stream);

/* Bytes of the chunk states ss_ssd_fwd saves in ckpt: batch * nheads *
 * ceil(seqlen / 64) * dstate * headdim * 4 (0 for empty shapes). */
size_t ss_ssd_ckpt_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                        int64_t dstate);

/* Bytes of device workspace ss_ssd_bwd needs (0 for empty shapes). */
size_t ss_ssd_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                 int64_t ngroups, int64_t dstate);

/*
 * Mamba-2 SSD backward: gradients of sum(dout * out) + sum(dlast * last_state)
 * for ss_ssd_fwd with the same arguments (same shapes, dtypes and limits).
 *   dout           (batch, seqlen, nheads, headdim) bf16, required
 *   dlast          (batch, nheads, headdim, dstate) f32 or NULL
 *   dx             like x, bf16, required
 *   ddt            like dt, bf16, required (w.r.t. the raw dt)
 *   dA             (nheads) f32, required; summed over batch and time
 *   dB, dC         like B, C, bf16, required; summed over the group's heads
 *   dD, ddt_bias   NULL iff D / dt_bias is NULL
 *   dh0            optional (may be given without h0: the gradient at a zero start)
 *   ckpt           what ss_ssd_fwd saved for exactly these inputs, or NULL (then
 *                  the states are recomputed in the workspace)
 *   workspace      ss_ssd_bwd_workspace_size() bytes, 16-byte aligned; it holds
 *                  the state entering every chunk of 64 steps (f32), the
 *                  per-head dB / dC terms (f32) and per-step partials, about
 *                  4 * batch * nheads * ceil(seqlen / 64) * 64 * dstate *
 *                  (headdim / 64 + 2) bytes
 * The gradients are taken in the same chunked form as the forward
 * (back-propagation through time regrouped by chunk, on bf16 matrix cores
 * with f32 accumulation): a states pass (unless ckpt), one reverse pass per (batch, head)
 * carrying the state's adjoint, then the suffix sums that give ddt and dA,
 * and the sums of dB, dC over each group's heads.  Every sum runs in a fixed
 * order: results are deterministic and do not depend on the batch size.
 * Besides ss_ssd_fwd's limits: batch * nheads * ceil(seqlen / 64) <= 2^31 - 1
 * (SS_EUNSUPPORTED beyond).
 */
ss_status ss_ssd_bwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                     int64_t ngroups, int64_t dstate, int io_dtype, const void *x, const void *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const float *dt_bias, int dt_softplus, const float *h0, const void *dout,
                     const float *dlast, void *dx, void *ddt, float *dA, void *dB, void *dC,
                     float *dD, float *ddt_bias, float *dh0, const float *ckpt,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Profiling aid for callers that time the library's kernels one by one
 * (not needed for normal use).  When `events` is non-NULL, every later
 * ss_fwd / ss_bwd / ss_state_update / ss_conv1d_* / ss_ssd_* call on this thread records the next
 * unused entry of `events` (each a hipEvent_t created by the caller) on its
 * stream before its first kernel and after each kernel it launches, until
 * `count` entries are used.  ss_profile_events(NULL, 0) switches it off.
 * ss_profile_events_used() returns how many entries have been recorded.
 * Recording events does not change what the kernels compute.
 */
ss_status ss_profile_events(void **events, int count);
int ss_profile_events_used(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_H */
