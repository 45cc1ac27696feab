/*
 * Selective state-space scan: the plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. The GPU library
 * shares no code, header, table or helper with it, and neither includes the
 * other.
 *
 * What it computes, and where the pages say so
 * (page "Mamba and State Space Models", world.lapla.si):
 *   - section "A State of Fixed Size": each input updates a fixed-size state,
 *     h <- Abar*h + Bbar*x, and the output is read as y = C*h, after the
 *     update;
 *   - section "Chosen by the Token": Delta, B and C are per-token inputs, A is
 *     fixed, and the share of the old state that stays is exp(Delta*A);
 *   - section "Taken Apart": one token moves the state once, which is the
 *     single-token decode update (oracle_state_update is the scan with L = 1).
 * Steps the pages leave open, each taken in its plainest reading:
 *   - the input discretisation is the first-order (Euler) form
 *     Bbar = Delta*B; a zero-order-hold form Bbar = (exp(Delta*A)-1)/A * B is
 *     available through `zoh` only so a test can check the gate identity of
 *     the paper's Theorem 1 (section "Chosen by the Token");
 *   - the skip term D*x is added to C*h before the output gate, and the gate
 *     multiplies by silu(z) = z / (1 + exp(-z));
 *   - one B and one C per (batch, token), shared by all channels;
 *   - optionally delta arrives before its activation: a per-channel bias is
 *     added and softplus(v) = log(1 + exp(v)) applied (the pages say delta
 *     comes from a projection of the token and must be positive; softplus is
 *     the activation the workloads use to make it so).
 *
 * Layout (row-major): x, delta, z, y are (batch, L, dim) with dim contiguous;
 * B and C are (batch, L, dstate); A is (dim, dstate); Dskip and delta_bias
 * are (dim); h0 and hL are (batch, dim, dstate). Every array is fp64. Dskip,
 * z, h0, hL and delta_bias may be NULL (no skip, no gate, zero initial
 * state, no final state, no bias).
 *
 * Nothing is blocked, fused or reordered: for each (batch, channel) the loop
 * runs token by token and state by state, exactly as the recurrence is
 * written. Channels are independent, so the (batch, channel) loop runs under
 * OpenMP; the arithmetic of each channel is the same sequential loop.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_DSTATE 256

/* Status codes: 0 ok, -1 invalid argument. */
int oracle_max_dstate(void) { return ORACLE_MAX_DSTATE; }

/* softplus(v) = log(1 + exp(v)), written so exp never overflows */
static double softplus(double v)
{
    return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));
}

int oracle_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, const double* h0, double* y, double* hL,
                    int zoh, const double* delta_bias, int delta_softplus)
{
    if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > ORACLE_MAX_DSTATE)
        return -1;
    if (batch == 0 || dim == 0) return 0;
    if (seqlen > 0 && (!x || !delta || !Bm || !Cm || !y)) return -1;
    if (!A) return -1;

    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            double h[ORACLE_MAX_DSTATE];
            /* the state before the first token */
            for (int64_t n = 0; n < dstate; ++n)
                h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;

            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t i_tok = (b * seqlen + t) * dim + d;  /* (b, t, d) */
                const int64_t i_bc = (b * seqlen + t) * dstate;    /* (b, t, 0) */
                double dt = delta[i_tok];
                const double u = x[i_tok];
                if (delta_bias) dt += delta_bias[d];
                if (delta_softplus) dt = softplus(dt);

                /* h <- Abar*h + Bbar*x, then read out y = C*h */
                double out = 0.0;
                for (int64_t n = 0; n < dstate; ++n) {
                    const double a = A[d * dstate + n];
                    const double Abar = exp(dt * a);
                    const double Bbar = zoh ? (Abar - 1.0) / a * Bm[i_bc + n]
                                            : dt * Bm[i_bc + n];
                    h[n] = Abar * h[n] + Bbar * u;
                    out += Cm[i_bc + n] * h[n];
                }
                if (Dskip) out += Dskip[d] * u;
                if (z) {
                    const double zz = z[i_tok];
                    out *= zz / (1.0 + exp(-zz));
                }
                y[i_tok] = out;
            }

            if (hL)
                for (int64_t n = 0; n < dstate; ++n)
                    hL[(b * dim + d) * dstate + n] = h[n];
        }
    }
    return 0;
}

/*
 * Single-token decode: one step of the same recurrence, with the state read
 * from h and written back to h. By definition it equals the scan over one
 * token with h0 = hL = h.
 */
int oracle_state_update(int64_t batch, int64_t dim, int64_t dstate, double* h,
                        const double* x, const double* delta, const double* A,
                        const double* Bm, const double* Cm, const double* Dskip,
                        const double* z, double* y, const double* delta_bias,
                        int delta_softplus)
{
    if (!h) return -1;
    return oracle_scan_fwd(batch, 1, dim, dstate, x, delta, A, Bm, Cm, Dskip, z,
                           h, y, h, 0, delta_bias, delta_softplus);
}

/*
 * Short causal convolution of the Mamba block (page "Mamba and State Space
 * Models", section "A State of Fixed Size": besides the SSM state each
 * channel keeps a short convolution over its last 4 inputs; the podcast page
 * and the dictionary page name the same short convolution as part of the
 * block). The pages give no formula; the plainest reading, used here:
 *
 *   pre[b,t,d] = bias[d] + sum_{k=0}^{W-1} weight[d,k] * x[b, t-(W-1)+k, d]
 *   y[b,t,d]   = silu(pre) if `silu`, else pre
 *
 * i.e. each channel is filtered on its own (depthwise) and only the current
 * and the W-1 previous inputs are seen (causal); weight[d, W-1] multiplies
 * the current token. Inputs before the first token come from `state_in`, the
 * last W inputs of whatever preceded the sequence (state_in[b,d,W-1] is the
 * newest), or are zero when it is NULL. `state_out` receives the last W
 * inputs as the sequence leaves them, in the same layout, so the next call
 * (or the next decode step) continues the sequence exactly.
 *
 * Layout: x, y (batch, L, dim), dim contiguous; weight (dim, W); bias (dim)
 * or NULL; state_in, state_out (batch, dim, W) or NULL. Every array is fp64.
 * state_out may alias state_in.
 */
static double conv_input(const double* x, const double* carried, int64_t b, int64_t s,
                         int64_t d, int64_t seqlen, int64_t dim, int64_t width)
{
    /* input s of channel (b, d); s < 0 reaches into the W carried inputs */
    if (s >= 0) return x[(b * seqlen + s) * dim + d];
    return carried[width + s];
}

int oracle_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                      const double* x, const double* weight, const double* bias,
                      const double* state_in, double* y, double* state_out, int silu)
{
    if (batch < 0 || seqlen < 0 || dim < 0 || width < 1 || width > 64) return -1;
    if (batch == 0 || dim == 0) return 0;
    if (!weight || (seqlen > 0 && (!x || !y))) return -1;

    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            /* copied first, so state_out may alias state_in */
            double carried[64];
            for (int64_t k = 0; k < width; ++k)
                carried[k] = state_in ? state_in[(b * dim + d) * width + k] : 0.0;

            for (int64_t t = 0; t < seqlen; ++t) {
                double pre = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < width; ++k)
                    pre += weight[d * width + k] *
                           conv_input(x, carried, b, t - (width - 1) + k, d, seqlen, dim, width);
                y[(b * seqlen + t) * dim + d] = silu ? pre / (1.0 + exp(-pre)) : pre;
            }
            if (state_out)
                for (int64_t k = 0; k < width; ++k)
                    state_out[(b * dim + d) * width + k] =
                        conv_input(x, carried, b, seqlen - width + k, d, seqlen, dim, width);
        }
    }
    return 0;
}

/*
 * Decode step of the short convolution: the new input joins the W carried
 * inputs (the oldest drops out) and one output is produced. By definition
 * the forward convolution over one token with state_in = state_out = state.
 * x, y (batch, dim); state (batch, dim, W), updated in place.
 */
int oracle_conv1d_update(int64_t batch, int64_t dim, int64_t width, double* state,
                         const double* x, const double* weight, const double* bias,
                         double* y, int silu)
{
    if (!state) return -1;
    return oracle_conv1d_fwd(batch, 1, dim, width, x, weight, bias, state, y, state, silu);
}

/*
 * Backward pass of the scan (page "Mamba and State Space Models", section
 * "A Scan on the Chip": training's backward pass needs the intermediate
 * states, which are computed again rather than stored). This oracle simply
 * keeps every state of a channel while it runs the forward recurrence once
 * more, then walks the sequence backwards applying the chain rule to each
 * step of oracle_scan_fwd.
 *
 * The loss is L = sum(dy * y) + sum(dhL * hL): dy (batch, L, dim) is the
 * gradient arriving at y, dhL (batch, dim, dstate) the one arriving at the
 * final state (NULL: zero). With the state's adjoint
 *   lam_t[n] = dL/dh_t[n] = C_t[n] * g_t + Abar_{t+1}[n] * lam_{t+1}[n],
 *   lam_{L-1}[n] = C_{L-1}[n] * g_{L-1} + dhL[n],   g_t = dy_t * silu(z_t),
 * the gradients of one step h_t = Abar_t h_{t-1} + dt_t B_t x_t,
 * Abar_t = exp(dt_t A), are
 *   dx_t     = D g_t + sum_n lam_t[n] dt_t B_t[n]
 *   d dt_t   = sum_n lam_t[n] (A[n] Abar_t[n] h_{t-1}[n] + B_t[n] x_t)
 *   dA[n]   += lam_t[n] dt_t Abar_t[n] h_{t-1}[n]
 *   dB_t[n] += lam_t[n] dt_t x_t        (summed over channels)
 *   dC_t[n] += g_t h_t[n]               (summed over channels)
 *   dD      += g_t x_t
 *   dz_t     = dy_t p_t silu'(z_t),  p_t = C_t . h_t + D x_t,
 *              silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + exp(-z))
 *   dh0[n]   = Abar_0[n] lam_0[n]
 * and with the fused activation dt = softplus(v), v = delta + bias:
 *   d delta = d dt * sigmoid(v),  d bias += d delta.
 * dA, dD and d bias sum over batch rows; dB and dC over channels. Outputs
 * are fp64 and overwritten: dx, ddelta, dz (batch, L, dim); dB, dC
 * (batch, L, dstate); dA (dim, dstate); dD, ddelta_bias (dim); dh0
 * (batch, dim, dstate). dD, dz, dh0, ddelta_bias may be NULL (not wanted);
 * dz must be NULL when z is, dD when Dskip is, ddelta_bias when delta_bias is.
 * Batch rows run in parallel; everything within a row runs in order, and the
 * sums over rows are taken in row order afterwards.
 */
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

int oracle_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    const double* x, const double* delta, const double* A,
                    const double* Bm, const double* Cm, const double* Dskip,
                    const double* z, const double* h0, const double* delta_bias,
                    int delta_softplus, const double* dy, const double* dhL,
                    double* dx, double* ddelta, double* dA, double* dB, double* dC,
                    double* dD, double* dz, double* dh0, double* ddelta_bias)
{
    if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > ORACLE_MAX_DSTATE)
        return -1;
    if (!A || !dA) return -1;
    if (seqlen > 0 && (!x || !delta || !Bm || !Cm || !dy || !dx || !ddelta || !dB || !dC))
        return -1;
    if ((dz && !z) || (dD && !Dskip) || (ddelta_bias && !delta_bias)) return -1;

    const int64_t N = dstate;
    memset(dA, 0, sizeof(double) * (size_t)(dim * N));
    if (dD) memset(dD, 0, sizeof(double) * (size_t)dim);
    if (ddelta_bias) memset(ddelta_bias, 0, sizeof(double) * (size_t)dim);
    if (batch == 0 || dim == 0) return 0;
    if (seqlen > 0) {
        memset(dB, 0, sizeof(double) * (size_t)(batch * seqlen * N));
        memset(dC, 0, sizeof(double) * (size_t)(batch * seqlen * N));
    }
    /* per-row partial sums of dA, dD, d bias, added up in row order below */
    double* pA = calloc((size_t)(batch * dim * N), sizeof(double));
    double* pD = calloc((size_t)(batch * dim), sizeof(double));
    double* pBias = calloc((size_t)(batch * dim), sizeof(double));
    if (!pA || !pD || !pBias) {
        free(pA); free(pD); free(pBias);
        return -2;
    }
    int failed = 0;

    #pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        /* hs[(t + 1) * N + n] = h_t[n]; hs[n] = h_{-1} = h0 */
        double* hs = malloc(sizeof(double) * (size_t)((seqlen + 1) * N));
        double* dts = malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
        double* vs = malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
        if (!hs || !dts || !vs) {
            free(hs); free(dts); free(vs);
            #pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int64_t d = 0; d < dim; ++d) {
            /* forward once more, keeping every state */
            for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                const int64_t i_tok = (b * seqlen + t) * dim + d;
                const int64_t i_bc = (b * seqlen + t) * N;
                double v = delta[i_tok];
                if (delta_bias) v += delta_bias[d];
                const double dt = delta_softplus ? softplus(v) : v;
                vs[t] = v;
                dts[t] = dt;
                for (int64_t n = 0; n < N; ++n)
                    hs[(t + 1) * N + n] = exp(dt * A[d * N + n]) * hs[t * N + n] +
                                          dt * Bm[i_bc + n] * x[i_tok];
            }
            /* backwards through the steps */
            double lam[ORACLE_MAX_DSTATE];
            double abar_next[ORACLE_MAX_DSTATE];
            for (int64_t n = 0; n < N; ++n) {
                lam[n] = dhL ? dhL[(b * dim + d) * N + n] : 0.0;
                abar_next[n] = 1.0;
            }
            for (int64_t t = seqlen - 1; t >= 0; --t) {
                const int64_t i_tok = (b * seqlen + t) * dim + d;
                const int64_t i_bc = (b * seqlen + t) * N;
                const double u = x[i_tok];
                const double dt = dts[t];
                const double* h_now = hs + (t + 1) * N;
                const double* h_prev = hs + t * N;
                double s = 1.0, zz = 0.0;
                if (z) {
                    zz = z[i_tok];
                    s = sigmoid(zz);
                }
                const double gate = z ? zz * s : 1.0;
                const double g = dy[i_tok] * gate;  /* dL/dp_t */
                double p = Dskip ? Dskip[d] * u : 0.0;
                double dxt = Dskip ? Dskip[d] * g : 0.0;
                double ddt = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = A[d * N + n];
                    const double abar = exp(dt * a);
                    lam[n] = Cm[i_bc + n] * g + abar_next[n] * lam[n];
                    p += Cm[i_bc + n] * h_now[n];
                    dxt += lam[n] * dt * Bm[i_bc + n];
                    ddt += lam[n] * (a * abar * h_prev[n] + Bm[i_bc + n] * u);
                    pA[(b * dim + d) * N + n] += lam[n] * dt * abar * h_prev[n];
                    dB[i_bc + n] += lam[n] * dt * u;
                    dC[i_bc + n] += g * h_now[n];
                    abar_next[n] = abar;
                }
                if (dD) pD[b * dim + d] += g * u;
                if (dz) dz[i_tok] = dy[i_tok] * p * s * (1.0 + zz * (1.0 - s));
                dx[i_tok] = dxt;
                const double dv = delta_softplus ? ddt * sigmoid(vs[t]) : ddt;
                ddelta[i_tok] = dv;
                if (ddelta_bias) pBias[b * dim + d] += dv;
            }
            if (dh0)
                for (int64_t n = 0; n < N; ++n) dh0[(b * dim + d) * N + n] = abar_next[n] * lam[n];
        }
        free(hs);
        free(dts);
        free(vs);
    }
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < dim; ++d) {
            for (int64_t n = 0; n < N; ++n) dA[d * N + n] += pA[(b * dim + d) * N + n];
            if (dD) dD[d] += pD[b * dim + d];
            if (ddelta_bias) ddelta_bias[d] += pBias[b * dim + d];
        }
    free(pA);
    free(pD);
    free(pBias);
    return failed ? -2 : 0;
}

/*
 * Mamba-2's state space dual form (page "Mamba and State Space Models",
 * section "Mamba-2: Two Algorithms"): A is a number times the identity, so
 * the state of a channel decays by one factor exp(dt * a) for all its
 * states. The channels come in heads of `headdim` channels that share that
 * number a and the step dt, which is what lets a whole chunk be handled by
 * matrix products; B and C are shared by all heads. The result is exactly
 * the recurrence, so the oracle runs it token by token:
 *
 *   h[p,n] <- exp(dt a_h) h[p,n] + dt B[n] x[p],   y[p] = sum_n C[n] h[p,n]
 *   y[p]   = (y[p] + D[p] x[p]) * silu(z[p])
 *
 * Layout: x, z, y (batch, L, nheads*headdim), channel h*headdim + p
 * contiguous; dt (batch, L, nheads); A, dt_bias (nheads); B, C (batch, L,
 * dstate); Dskip (nheads*headdim); h0, hL (batch, nheads, headdim, dstate).
 * dt may arrive raw: dt_bias[h] is added and softplus applied when asked.
 */
int oracle_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, const double* x, const double* dt, const double* A,
                   const double* Bm, const double* Cm, const double* Dskip, const double* z,
                   const double* h0, double* y, double* hL, const double* dt_bias,
                   int dt_softplus)
{
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0 || dstate < 1 ||
        dstate > ORACLE_MAX_DSTATE)
        return -1;
    if (!A) return -1;
    if (batch == 0 || nheads == 0 || headdim == 0) return 0;
    if (seqlen > 0 && (!x || !dt || !Bm || !Cm || !y)) return -1;
    const int64_t dim = nheads * headdim;

    #pragma omp parallel for collapse(3) schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t hd = 0; hd < nheads; ++hd) {
            for (int64_t p = 0; p < headdim; ++p) {
                const int64_t d = hd * headdim + p;
                const int64_t row = (b * nheads + hd) * headdim + p;  /* (b, h, p) */
                double h[ORACLE_MAX_DSTATE];
                for (int64_t n = 0; n < dstate; ++n)
                    h[n] = h0 ? h0[row * dstate + n] : 0.0;
                for (int64_t t = 0; t < seqlen; ++t) {
                    double step = dt[(b * seqlen + t) * nheads + hd];
                    if (dt_bias) step += dt_bias[hd];
                    if (dt_softplus) step = softplus(step);
                    const double decay = exp(step * A[hd]);
                    const int64_t i_tok = (b * seqlen + t) * dim + d;
                    const int64_t i_bc = (b * seqlen + t) * dstate;
                    const double u = x[i_tok];
                    double out = 0.0;
                    for (int64_t n = 0; n < dstate; ++n) {
                        h[n] = decay * h[n] + step * Bm[i_bc + n] * u;
                        out += Cm[i_bc + n] * h[n];
                    }
                    if (Dskip) out += Dskip[d] * u;
                    if (z) out *= z[i_tok] / (1.0 + exp(-z[i_tok]));
                    y[i_tok] = out;
                }
                if (hL)
                    for (int64_t n = 0; n < dstate; ++n) hL[row * dstate + n] = h[n];
            }
        }
    }
    return 0;
}
