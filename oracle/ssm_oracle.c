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
