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
