/*
 * ss_oracle.c -- plain, sequential, double-precision reference of the Mamba
 * selective scan: forward, reverse-time backward and the one-token state
 * update.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this code.  The GPU library neither
 * includes, links nor calls it, and the two share no source, header, table
 * or helper.  Everything here is written for a reader to check by eye: one
 * row at a time, one time step at a time, one state index at a time, in
 * double precision, with no blocking, no fusion and no reordering.
 *
 * What is computed.  The state-spaces/mamba README (section "Usage",
 * subsection "Selective SSM") names the selective SSM layer of the Mamba
 * paper (its Section 3 and Algorithm 2) as the operation; the mamba-rs
 * README (section "Features") adds the full backward pass through the
 * recurrent state, and its "Quick start (CPU)" section the single-token
 * step on a carried state.  The pages print no formula.  The reading used
 * here is the input-dependent diagonal SSM with a zero-order-hold decay and
 * an Euler input term, per channel d and state index n:
 *
 *   delta_t  = delta_raw_t + bias[d]            (bias optional, else 0)
 *   delta_t  = softplus(delta_t)                (only if the flag is set)
 *   h_t[n]   = exp(delta_t * A[d,n]) * h_{t-1}[n] + delta_t * B_t[n] * u_t
 *   y_t      = (sum_n C_t[n] * h_t[n] + D[d] * u_t) * silu(z_t)
 *
 * with h_{-1} = h0 (zero when no initial state is given), silu(z) =
 * z * sigmoid(z), the gate applied only when z is given and the D term only
 * when D is given.  The bias enters the range of delta as the projection
 * bias the README's "Troubleshooting / Initialization" section describes.
 *
 * Layouts (row-major, contiguous):
 *   u, delta, z, y, dout, du, ddelta, dz : (nb, nd, nl)
 *   B, C, dB, dC                         : (nb, ns, nl)
 *   A, dA                                : (nd, ns)
 *   D, bias, dD, dbias                   : (nd)
 *   h0, last_state, dlast, dh0           : (nb, nd, ns)
 * where nb = batch, nd = channels (d_inner), ns = d_state, nl = sequence
 * length.  A "row" is one (b, d) pair, row index r = b * nd + d.
 *
 * Parity: pinned.  The tests check this file against closed forms (one
 * step, pure decay, geometric series), a brute-force time-invariant
 * convolution written independently, hand-derived worked examples, and
 * central finite differences / adjoint identities for the backward.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* softplus(x) = log(1 + exp(x)), evaluated without overflow. */
static double sso_softplus(double x)
{
    double ax = x < 0 ? -x : x;
    return (x > 0 ? x : 0.0) + log1p(exp(-ax));
}

/* sigmoid(x) = 1 / (1 + exp(-x)), evaluated without overflow. */
static double sso_sigmoid(double x)
{
    if (x >= 0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* delta after the optional bias and the optional softplus. */
static double sso_prep_delta(double raw, const double *bias, int64_t d, int softplus)
{
    double x = raw + (bias ? bias[d] : 0.0);
    return softplus ? sso_softplus(x) : x;
}

/*
 * Forward scan for rows [row_begin, row_end).
 * y (nb, nd, nl) is required; last_state (nb, nd, ns) may be NULL.
 */
void sso_fwd(int64_t nb, int64_t nd, int64_t ns, int64_t nl,
             const double *u, const double *delta, const double *A,
             const double *B, const double *C, const double *D,
             const double *z, const double *bias, int softplus,
             const double *h0, double *y, double *last_state,
             int64_t row_begin, int64_t row_end)
{
    (void)nb;
    double *h = (double *)malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1));
    if (!h) abort();
    for (int64_t r = row_begin; r < row_end; r++) {
        int64_t b = r / nd, d = r % nd;
        for (int64_t n = 0; n < ns; n++)
            h[n] = h0 ? h0[r * ns + n] : 0.0;
        for (int64_t t = 0; t < nl; t++) {
            double ut = u[r * nl + t];
            double dt = sso_prep_delta(delta[r * nl + t], bias, d, softplus);
            double acc = 0.0;
            for (int64_t n = 0; n < ns; n++) {
                double abar = exp(dt * A[d * ns + n]);
                double bt = B[(b * ns + n) * nl + t];
                h[n] = abar * h[n] + dt * bt * ut;
                acc += C[(b * ns + n) * nl + t] * h[n];
            }
            double ypre = acc + (D ? D[d] * ut : 0.0);
            if (z) {
                double zt = z[r * nl + t];
                ypre *= zt * sso_sigmoid(zt);
            }
            y[r * nl + t] = ypre;
        }
        if (last_state)
            for (int64_t n = 0; n < ns; n++)
                last_state[r * ns + n] = h[n];
    }
    free(h);
}

/*
 * Backward (reverse-time BPTT) of the loss  sum_{r,t} dout[r,t] * y[r,t]
 * (+ sum dlast * last_state when dlast is given) for batch entries
 * [b_begin, b_end).
 *
 * Per-step outputs du, ddelta (with respect to the raw delta argument) and
 * dz (when z is given) are written for the rows of those batch entries;
 * dB and dC are written for those batch entries (summed over every channel
 * d in ascending d).  dA, dD and dbias are ADDED to (the caller zeroes them
 * and, when it splits the batch, folds the pieces in ascending b); dh0 is
 * written when non-NULL.  Returns 0, or -1 if scratch memory is unavailable.
 *
 * The adjoint g_t[n] = dLoss/dh_t[n] obeys, going backward in time,
 *   g_t = C_t * dy_t + exp(delta_{t+1} A) * g_{t+1},  g_{nl-1} seeded by dlast,
 * where dy_t = dout_t * silu(z_t) is the gradient at the pre-gate output.
 */
int sso_bwd(int64_t nb, int64_t nd, int64_t ns, int64_t nl,
            const double *u, const double *delta, const double *A,
            const double *B, const double *C, const double *D,
            const double *z, const double *bias, int softplus,
            const double *h0, const double *dout, const double *dlast,
            double *du, double *ddelta, double *dA, double *dB, double *dC,
            double *dD, double *dz, double *dbias, double *dh0,
            int64_t b_begin, int64_t b_end)
{
    (void)nb;
    size_t nsz = (size_t)(ns > 0 ? ns : 1);
    size_t nlz = (size_t)(nl > 0 ? nl : 1);
    double *hs = (double *)malloc(sizeof(double) * nsz * (nlz + 1)); /* h_{t-1} at hs[t*ns] */
    double *dl = (double *)malloc(sizeof(double) * nlz);
    double *g = (double *)malloc(sizeof(double) * nsz);
    if (!hs || !dl || !g) {
        free(hs); free(dl); free(g);
        return -1;
    }
    for (int64_t b = b_begin; b < b_end; b++) {
        for (int64_t n = 0; n < ns; n++)
            for (int64_t t = 0; t < nl; t++) {
                dB[(b * ns + n) * nl + t] = 0.0;
                dC[(b * ns + n) * nl + t] = 0.0;
            }
        for (int64_t d = 0; d < nd; d++) {
            int64_t r = b * nd + d;
            /* forward again, keeping every state: hs[(t+1)*ns + n] = h_t[n] */
            for (int64_t n = 0; n < ns; n++)
                hs[n] = h0 ? h0[r * ns + n] : 0.0;
            for (int64_t t = 0; t < nl; t++) {
                dl[t] = sso_prep_delta(delta[r * nl + t], bias, d, softplus);
                for (int64_t n = 0; n < ns; n++) {
                    double abar = exp(dl[t] * A[d * ns + n]);
                    hs[(t + 1) * ns + n] = abar * hs[t * ns + n]
                                         + dl[t] * B[(b * ns + n) * nl + t] * u[r * nl + t];
                }
            }
            /* backward in time */
            for (int64_t n = 0; n < ns; n++)
                g[n] = dlast ? dlast[r * ns + n] : 0.0;
            for (int64_t t = nl - 1; t >= 0; t--) {
                double ut = u[r * nl + t];
                double dout_t = dout[r * nl + t];
                const double *h_t = hs + (t + 1) * ns;
                const double *h_prev = hs + t * ns;
                double dy = dout_t;
                if (z) {
                    double ypre = D ? D[d] * ut : 0.0;
                    for (int64_t n = 0; n < ns; n++)
                        ypre += C[(b * ns + n) * nl + t] * h_t[n];
                    double zt = z[r * nl + t];
                    double s = sso_sigmoid(zt);
                    dy = dout_t * zt * s;
                    dz[r * nl + t] = dout_t * ypre * s * (1.0 + zt * (1.0 - s));
                }
                if (D) dD[d] += dy * ut;
                double sum_gb = 0.0, d_dt = 0.0;
                for (int64_t n = 0; n < ns; n++) {
                    double bt = B[(b * ns + n) * nl + t];
                    double ct = C[(b * ns + n) * nl + t];
                    double a = A[d * ns + n];
                    double abar = exp(dl[t] * a);
                    g[n] += ct * dy;                          /* g_t */
                    dC[(b * ns + n) * nl + t] += dy * h_t[n];
                    dB[(b * ns + n) * nl + t] += g[n] * dl[t] * ut;
                    sum_gb += g[n] * bt;
                    d_dt += g[n] * (a * abar * h_prev[n] + bt * ut);
                    dA[d * ns + n] += g[n] * dl[t] * abar * h_prev[n];
                    g[n] *= abar;                             /* carried to t-1 */
                }
                du[r * nl + t] = dl[t] * sum_gb + (D ? D[d] * dy : 0.0);
                double raw_grad = d_dt;
                if (softplus)
                    raw_grad *= sso_sigmoid(delta[r * nl + t] + (bias ? bias[d] : 0.0));
                ddelta[r * nl + t] = raw_grad;
                if (bias) dbias[d] += raw_grad;
            }
            if (dh0)
                for (int64_t n = 0; n < ns; n++)
                    dh0[r * ns + n] = g[n];
        }
    }
    free(hs); free(dl); free(g);
    return 0;
}

/*
 * One-token state update for rows [row_begin, row_end): the forward
 * recurrence advanced by a single step from the carried state, which is
 * overwritten in place (mamba-rs README, "Quick start (CPU)": the step call
 * on a carried MambaState).
 *   u, delta, z, y : (nb, nd);  B, C : (nb, ns);  state : (nb, nd, ns).
 */
void sso_state_update(int64_t nb, int64_t nd, int64_t ns,
                      double *state, const double *u, const double *delta,
                      const double *A, const double *B, const double *C,
                      const double *D, const double *z, const double *bias,
                      int softplus, double *y, int64_t row_begin, int64_t row_end)
{
    (void)nb;
    for (int64_t r = row_begin; r < row_end; r++) {
        int64_t b = r / nd, d = r % nd;
        double ut = u[r];
        double dt = sso_prep_delta(delta[r], bias, d, softplus);
        double acc = 0.0;
        for (int64_t n = 0; n < ns; n++) {
            double abar = exp(dt * A[d * ns + n]);
            double *h = state + r * ns + n;
            *h = abar * *h + dt * B[b * ns + n] * ut;
            acc += C[b * ns + n] * *h;
        }
        double ypre = acc + (D ? D[d] * ut : 0.0);
        if (z) ypre *= z[r] * sso_sigmoid(z[r]);
        y[r] = ypre;
    }
}

/* ------------------------------------------------------------------------
 * Causal depthwise convolution over time, optionally followed by SiLU.
 *
 * The state-spaces/mamba README's Mamba block ("Usage / Mamba Block")
 * configures a local convolution of width d_conv (4) in front of the
 * selective SSM, and the mamba-rs README's "Quick start (CPU)" carries its
 * window in the decoding state (MambaState::zeros(..., d_conv)).  Neither
 * page prints the operation; the reading used here is the causal, per
 * channel (depthwise) convolution of width K, with SiLU applied when asked:
 *
 *   pre_t = bias[d] + sum_{k=0}^{K-1} w[d,k] * x_{t-(K-1)+k}
 *   out_t = silu(pre_t)  (or pre_t)
 *
 * where the inputs before t = 0 come from an initial window s0[b,d,j] =
 * x_{j-(K-1)} (j = 0..K-2), zero when no window is given.  The final window
 * is x_{L-(K-1)+j}, j = 0..K-2 (entries before t = 0 again from s0 or 0).
 * The decode update steps that window by one input.
 *
 * Layouts: x, out, dout, dx (nb, nd, nl); w, dw (nd, nk); bias, dbias (nd);
 *          s0, s_final, ds0, decode state (nb, nd, nk - 1); decode x, out
 *          (nb, nd).
 * ------------------------------------------------------------------------ */

/* x_tt of row r, tt in [-(nk-1), nl): from x, or from the initial window */
static double sso_conv_in(const double *x, const double *s0, int64_t r, int64_t nl,
                          int64_t nk, int64_t tt)
{
    if (tt >= 0) return x[r * nl + tt];
    return s0 ? s0[r * (nk - 1) + (tt + nk - 1)] : 0.0;
}

static double sso_conv_pre(const double *x, const double *w, const double *bias,
                           const double *s0, int64_t r, int64_t d, int64_t nl, int64_t nk,
                           int64_t t)
{
    double acc = bias ? bias[d] : 0.0;
    for (int64_t k = 0; k < nk; k++)
        acc += w[d * nk + k] * sso_conv_in(x, s0, r, nl, nk, t - (nk - 1) + k);
    return acc;
}

/* rows r0 <= r < r1 */
void sso_conv_fwd(int64_t nb, int64_t nd, int64_t nl, int64_t nk,
                  const double *x, const double *w, const double *bias, int silu,
                  const double *s0, double *out, double *s_final, int64_t r0, int64_t r1)
{
    (void)nb;
    for (int64_t r = r0; r < r1; r++) {
        int64_t d = r % nd;
        for (int64_t t = 0; t < nl; t++) {
            double pre = sso_conv_pre(x, w, bias, s0, r, d, nl, nk, t);
            out[r * nl + t] = silu ? pre * sso_sigmoid(pre) : pre;
        }
        if (s_final)
            for (int64_t j = 0; j < nk - 1; j++)
                s_final[r * (nk - 1) + j] = sso_conv_in(x, s0, r, nl, nk, nl - (nk - 1) + j);
    }
}

/*
 * Backward of sum(dout * out).  With g_t = dout_t * silu'(pre_t) (or dout_t),
 * silu'(p) = s (1 + p (1 - s)), s = sigmoid(p):
 *   dx_tt   = sum over (t, k) with t - (K-1) + k = tt of w[d,k] g_t
 *   ds0_j   = the same sum for tt = j - (K-1) < 0
 *   dw[d,k] = sum_{b,t} g_t x_{t-(K-1)+k},   dbias[d] = sum_{b,t} g_t
 * Batch entries b0 <= b < b1; dw and dbias are accumulated (the caller
 * zeroes them), over b, then t, ascending.
 */
void sso_conv_bwd(int64_t nb, int64_t nd, int64_t nl, int64_t nk,
                  const double *x, const double *w, const double *bias, int silu,
                  const double *s0, const double *dout, double *dx, double *dw,
                  double *dbias, double *ds0, int64_t b0, int64_t b1)
{
    (void)nb;
    for (int64_t b = b0; b < b1; b++) {
        for (int64_t d = 0; d < nd; d++) {
            int64_t r = b * nd + d;
            for (int64_t t = 0; t < nl; t++) dx[r * nl + t] = 0.0;
            if (ds0)
                for (int64_t j = 0; j < nk - 1; j++) ds0[r * (nk - 1) + j] = 0.0;
            for (int64_t t = 0; t < nl; t++) {
                double pre = sso_conv_pre(x, w, bias, s0, r, d, nl, nk, t);
                double g = dout[r * nl + t];
                if (silu) {
                    double s = sso_sigmoid(pre);
                    g *= s * (1.0 + pre * (1.0 - s));
                }
                if (dbias) dbias[d] += g;
                for (int64_t k = 0; k < nk; k++) {
                    int64_t tt = t - (nk - 1) + k;
                    dw[d * nk + k] += g * sso_conv_in(x, s0, r, nl, nk, tt);
                    if (tt >= 0)
                        dx[r * nl + tt] += w[d * nk + k] * g;
                    else if (ds0)
                        ds0[r * (nk - 1) + (tt + nk - 1)] += w[d * nk + k] * g;
                }
            }
        }
    }
}

/* One input per row: out = silu(bias + sum_k w[k] window_k) with window =
 * (state[0..K-2], x); the state then drops its oldest entry and takes x. */
void sso_conv_update(int64_t nb, int64_t nd, int64_t nk, double *state, const double *x,
                     const double *w, const double *bias, int silu, double *out)
{
    for (int64_t r = 0; r < nb * nd; r++) {
        int64_t d = r % nd;
        double acc = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < nk; k++) {
            double v = (k < nk - 1) ? state[r * (nk - 1) + k] : x[r];
            acc += w[d * nk + k] * v;
        }
        out[r] = silu ? acc * sso_sigmoid(acc) : acc;
        for (int64_t j = 0; j < nk - 1; j++)
            state[r * (nk - 1) + j] = (j + 1 < nk - 1) ? state[r * (nk - 1) + j + 1] : x[r];
    }
}

/* ------------------------------------------------------------------------
 * Mamba-2 SSD: the selective scan with a scalar A per head.
 *
 * The state-spaces/mamba README ("Mamba-2", "SSD") names the Mamba-2 block
 * and its inner SSD module with d_state typically 64 or 128; the pages print
 * no formula.  The reading: per batch b and head h, a state H of headdim x
 * d_state entries,
 *
 *   dt_t   = softplus(dt_raw[b,t,h] + dt_bias[h])      (bias, softplus optional)
 *   H_t    = exp(dt_t A[h]) H_{t-1} + dt_t x_t B_t^T     (x_t: headdim, B_t: d_state)
 *   y_t    = H_t C_t + D[h] x_t
 *
 * with B, C shared by the heads of a group (group = h / (nheads / ngroups))
 * and H_{-1} = h0 (zero without one).  Layouts (time-major, as the mamba-rs
 * scratch buffers of the Mamba-3 block lay out their per-step tensors):
 * x, y (nb, nl, nh, np); dt (nb, nl, nh); B, C (nb, nl, ng, ns);
 * A, D, dt_bias (nh); h0, last (nb, nh, np, ns).
 * (b, h) pairs with b0 <= b < b1 are computed.
 * ------------------------------------------------------------------------ */
int sso_ssd_fwd(int64_t nb, int64_t nl, int64_t nh, int64_t np, int64_t ng, int64_t ns,
                const double *x, const double *dtr, const double *A, const double *B,
                const double *C, const double *D, const double *dt_bias, int softplus,
                const double *h0, double *y, double *last, int64_t b0, int64_t b1)
{
    (void)nb;
    double *H = (double *)malloc(sizeof(double) * (size_t)(np * ns > 0 ? np * ns : 1));
    if (!H) return 1;
    for (int64_t b = b0; b < b1; b++) {
        for (int64_t h = 0; h < nh; h++) {
            const int64_t g = h / (nh / ng);
            for (int64_t i = 0; i < np * ns; i++)
                H[i] = h0 ? h0[(b * nh + h) * np * ns + i] : 0.0;
            for (int64_t t = 0; t < nl; t++) {
                double dt = dtr[(b * nl + t) * nh + h] + (dt_bias ? dt_bias[h] : 0.0);
                if (softplus) dt = sso_softplus(dt);
                const double decay = exp(dt * A[h]);
                const double *xt = x + ((b * nl + t) * nh + h) * np;
                const double *bt = B + ((b * nl + t) * ng + g) * ns;
                const double *ct = C + ((b * nl + t) * ng + g) * ns;
                double *yt = y + ((b * nl + t) * nh + h) * np;
                for (int64_t p = 0; p < np; p++) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < ns; n++) {
                        double *hv = &H[p * ns + n];
                        *hv = decay * *hv + dt * xt[p] * bt[n];
                        acc += ct[n] * *hv;
                    }
                    yt[p] = acc + (D ? D[h] * xt[p] : 0.0);
                }
            }
            if (last)
                for (int64_t i = 0; i < np * ns; i++) last[(b * nh + h) * np * ns + i] = H[i];
        }
    }
    free(H);
    return 0;
}

/*
 * Backward of sum(dy * y) + sum(dlast * H_last) for sso_ssd_fwd, by
 * back-propagation through time.  With G_t = dL/dH_t (headdim x d_state),
 *   G_t      = dlast (t = L-1) or exp(dt_{t+1} A) G_{t+1}, plus dy_t C_t^T
 *   dx_t     = dt_t G_t B_t + D dy_t
 *   dB_t    += dt_t G_t^T x_t          (summed over the heads of the group)
 *   dC_t    += H_t^T dy_t              (likewise)
 *   d dt_t   = < G_t, A exp(dt_t A) H_{t-1} + x_t B_t^T >
 *   dA      += dt_t exp(dt_t A) < G_t, H_{t-1} >
 *   dD      += < x_t, dy_t >
 *   dh0      = exp(dt_0 A) G_0
 * and the raw dt gets d dt_t times softplus'(raw) = sigmoid(raw) when
 * softplus is on; d dt_bias sums it.  dA, dD, ddt_bias, dB, dC accumulate
 * (the caller zeroes them); batches b0 <= b < b1.
 */
int sso_ssd_bwd(int64_t nb, int64_t nl, int64_t nh, int64_t np, int64_t ng, int64_t ns,
                const double *x, const double *dtr, const double *A, const double *B,
                const double *C, const double *D, const double *dt_bias, int softplus,
                const double *h0, const double *dy, const double *dlast, double *dx,
                double *ddt, double *dA, double *dB, double *dC, double *dD, double *ddt_bias,
                double *dh0, int64_t b0, int64_t b1)
{
    (void)nb;
    const int64_t ps = np * ns;
    double *Hs = (double *)malloc(sizeof(double) * (size_t)(ps > 0 ? ps : 1) * (size_t)(nl + 1));
    double *Gs = (double *)malloc(sizeof(double) * (size_t)(ps > 0 ? ps : 1));
    double *dtv = (double *)malloc(sizeof(double) * (size_t)(nl > 0 ? nl : 1));
    if (!Hs || !Gs || !dtv) { free(Hs); free(Gs); free(dtv); return 1; }
    for (int64_t b = b0; b < b1; b++) {
        for (int64_t h = 0; h < nh; h++) {
            const int64_t g = h / (nh / ng);
            /* forward states H_{-1} .. H_{L-1} at Hs[(t + 1) * ps] */
            for (int64_t i = 0; i < ps; i++) Hs[i] = h0 ? h0[(b * nh + h) * ps + i] : 0.0;
            for (int64_t t = 0; t < nl; t++) {
                double dt = dtr[(b * nl + t) * nh + h] + (dt_bias ? dt_bias[h] : 0.0);
                if (softplus) dt = sso_softplus(dt);
                dtv[t] = dt;
                const double a = exp(dt * A[h]);
                const double *xt = x + ((b * nl + t) * nh + h) * np;
                const double *bt = B + ((b * nl + t) * ng + g) * ns;
                for (int64_t p = 0; p < np; p++)
                    for (int64_t n = 0; n < ns; n++)
                        Hs[(t + 1) * ps + p * ns + n] = a * Hs[t * ps + p * ns + n] + dt * xt[p] * bt[n];
            }
            for (int64_t i = 0; i < ps; i++) Gs[i] = dlast ? dlast[(b * nh + h) * ps + i] : 0.0;
            for (int64_t t = nl - 1; t >= 0; t--) {
                const double dt = dtv[t], a = exp(dt * A[h]);
                const double *xt = x + ((b * nl + t) * nh + h) * np;
                const double *bt = B + ((b * nl + t) * ng + g) * ns;
                const double *ct = C + ((b * nl + t) * ng + g) * ns;
                const double *dyt = dy + ((b * nl + t) * nh + h) * np;
                double *dxt = dx + ((b * nl + t) * nh + h) * np;
                double *dbt = dB + ((b * nl + t) * ng + g) * ns;
                double *dct = dC + ((b * nl + t) * ng + g) * ns;
                const double *Ht = Hs + (t + 1) * ps, *Hp = Hs + t * ps;
                double d_dt = 0.0, d_a = 0.0;
                for (int64_t p = 0; p < np; p++) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < ns; n++) {
                        double *gv = &Gs[p * ns + n];
                        *gv += dyt[p] * ct[n];                /* G_t */
                        acc += *gv * bt[n];
                        dbt[n] += dt * *gv * xt[p];
                        dct[n] += Ht[p * ns + n] * dyt[p];
                        d_dt += *gv * xt[p] * bt[n];
                        d_a += *gv * Hp[p * ns + n];
                    }
                    dxt[p] = dt * acc + (D ? D[h] * dyt[p] : 0.0);
                    if (dD) dD[h] += xt[p] * dyt[p];
                }
                d_dt += A[h] * a * d_a;
                dA[h] += dt * a * d_a;
                double raw_grad = d_dt;
                if (softplus)
                    raw_grad *= sso_sigmoid(dtr[(b * nl + t) * nh + h] + (dt_bias ? dt_bias[h] : 0.0));
                ddt[(b * nl + t) * nh + h] = raw_grad;
                if (ddt_bias) ddt_bias[h] += raw_grad;
                for (int64_t i = 0; i < ps; i++) Gs[i] *= a;   /* carried to t - 1 */
            }
            if (dh0)
                for (int64_t i = 0; i < ps; i++) dh0[(b * nh + h) * ps + i] = Gs[i];
        }
    }
    free(Hs); free(Gs); free(dtv);
    return 0;
}
