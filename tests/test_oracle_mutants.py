"""Planted mistakes in the oracle must be caught by its pins.

Each mutant rewrites one spot of oracle/ssm_oracle.c (a dropped term, a wrong
sign, a wrong or transposed index, a swapped operand), compiles the result
into a temporary library on the CPU and runs every pin against it: at least
one pin must fail. The real oracle source is never modified.
"""
import os

import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

MUTANTS = {
    "decay sign flipped": ("const double Abar = exp(dt * a);", "const double Abar = exp(-dt * a);"),
    "delta dropped from Bbar": (": dt * Bm[i_bc + n];", ": Bm[i_bc + n];"),
    "decay of h dropped": ("Abar * h[n] + Bbar * u", "h[n] + Bbar * u"),
    "readout uses B": ("h[n] = Abar * h[n] + Bbar * u;\n                    out += Cm[i_bc + n] * h[n];",
                       "h[n] = Abar * h[n] + Bbar * u;\n                    out += Bm[i_bc + n] * h[n];"),
    "A transposed": ("const double a = A[d * dstate + n];", "const double a = A[n * dim + d];"),
    "skip term dropped": ("if (Dskip) out += Dskip[d] * u;\n                if (z) {", "if (z) {"),
    "gate sign flipped": ("out *= zz / (1.0 + exp(-zz));", "out *= zz / (1.0 + exp(zz));"),
    "h0 ignored": ("h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;", "h[n] = 0.0;"),
    "readout before update": (
        "h[n] = Abar * h[n] + Bbar * u;\n                    out += Cm[i_bc + n] * h[n];",
        "out += Cm[i_bc + n] * h[n];\n                    h[n] = Abar * h[n] + Bbar * u;"),
    "B, C from the previous token": ("const int64_t i_bc = (b * seqlen + t) * dstate;    /*",
                                     "const int64_t i_bc = (b * seqlen + (t > 0 ? t - 1 : 0)) * dstate;    /*"),
    "B, C ignore the batch": ("const int64_t i_bc = (b * seqlen + t) * dstate;    /*",
                              "const int64_t i_bc = t * dstate;    /*"),
    "x from the previous token": (
        "const double u = x[i_tok];\n                if (delta_bias)",
        "const double u = x[i_tok - (t > 0 ? dim : 0)];\n                if (delta_bias)"),
    "x and delta swapped": ("double dt = delta[i_tok];\n                const double u = x[i_tok];",
                            "double dt = x[i_tok];\n                const double u = delta[i_tok];"),
    "delta bias ignored": ("if (delta_bias) dt += delta_bias[d];", ""),
    "delta bias after the activation": (
        "if (delta_bias) dt += delta_bias[d];\n                if (delta_softplus) dt = softplus(dt);",
        "if (delta_softplus) dt = softplus(dt);\n                if (delta_bias) dt += delta_bias[d];"),
    "softplus sign": ("return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));",
                      "return v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(-v));"),
    "softplus dropped": ("if (delta_softplus) dt = softplus(dt);",
                         "if (delta_softplus) dt = softplus(dt) * 0.0 + dt;"),
    "final state scaled": ("hL[(b * dim + d) * dstate + n] = h[n];",
                           "hL[(b * dim + d) * dstate + n] = 0.5 * h[n];"),
    "zero-order hold sign": ("(Abar - 1.0) / a", "(1.0 - Abar) / a"),
    "skip uses the wrong channel": ("if (Dskip) out += Dskip[d] * u;\n                if (z) {",
                                    "if (Dskip) out += Dskip[dim - 1 - d] * u;\n                if (z) {"),
    "conv taps reversed": ("pre += weight[d * width + k] *",
                           "pre += weight[d * width + (width - 1 - k)] *"),
    "conv taps shifted by one token": ("conv_input(x, carried, b, t - (width - 1) + k, d,",
                                       "conv_input(x, carried, b, t - width + k, d,"),
    "conv carried inputs newest first": ("return carried[width + s];", "return carried[-s - 1];"),
    "conv silu dropped": ("silu ? pre / (1.0 + exp(-pre)) : pre;", "pre;"),
    "conv bias dropped": ("double pre = bias ? bias[d] : 0.0;", "double pre = 0.0;"),
    "conv state handed on one token early": ("conv_input(x, carried, b, seqlen - width + k, d,",
                                             "conv_input(x, carried, b, seqlen - width + k - 1, d,"),
    "bwd adjoint decays with this token's Abar": (
        "lam[n] = Cm[i_bc + n] * g + abar_next[n] * lam[n];",
        "lam[n] = Cm[i_bc + n] * g + abar * lam[n];"),
    "bwd final-state gradient ignored": ("lam[n] = dhL ? dhL[(b * dim + d) * N + n] : 0.0;",
                                         "lam[n] = 0.0;"),
    "bwd delta gradient drops the decay term": (
        "ddt += lam[n] * (a * abar * h_prev[n] + Bm[i_bc + n] * u);",
        "ddt += lam[n] * (Bm[i_bc + n] * u);"),
    "bwd dA uses the new state": ("pA[(b * dim + d) * N + n] += lam[n] * dt * abar * h_prev[n];",
                                  "pA[(b * dim + d) * N + n] += lam[n] * dt * abar * h_now[n];"),
    "bwd dB misses delta": ("dB[i_bc + n] += lam[n] * dt * u;", "dB[i_bc + n] += lam[n] * u;"),
    "bwd dC uses the previous state": ("dC[i_bc + n] += g * h_now[n];",
                                       "dC[i_bc + n] += g * h_prev[n];"),
    "bwd gate derivative wrong": ("s * (1.0 + zz * (1.0 - s))", "s * (1.0 - s)"),
    "bwd softplus derivative dropped": ("const double dv = delta_softplus ? ddt * sigmoid(vs[t]) : ddt;",
                                        "const double dv = ddt;"),
    "bwd dh0 misses the first decay": ("dh0[(b * dim + d) * N + n] = abar_next[n] * lam[n];",
                                       "dh0[(b * dim + d) * N + n] = lam[n];"),
    "bwd skip gradient dropped": ("double dxt = Dskip ? Dskip[d] * g : 0.0;", "double dxt = 0.0;"),
    "ssd decay from the next head": ("const double decay = exp(step * A[hd]);",
                                     "const double decay = exp(step * A[(hd + 1) % nheads]);"),
    "ssd dt from the first head": ("double step = dt[(b * seqlen + t) * nheads + hd];",
                                   "double step = dt[(b * seqlen + t) * nheads];"),
    "ssd B and C swapped": ("h[n] = decay * h[n] + step * Bm[i_bc + n] * u;\n                        out += Cm[i_bc + n] * h[n];",
                            "h[n] = decay * h[n] + step * Cm[i_bc + n] * u;\n                        out += Bm[i_bc + n] * h[n];"),
    "ssd state rows ignore the head": ("const int64_t row = (b * nheads + hd) * headdim + p;",
                                       "const int64_t row = b * nheads * headdim + p;"),
    "ssd decay applied twice": ("h[n] = decay * h[n] + step * Bm[i_bc + n] * u;",
                                "h[n] = decay * decay * h[n] + step * Bm[i_bc + n] * u;"),
    "ssd dt bias ignored": ("if (dt_bias) step += dt_bias[hd];", ""),
    "conv carried state ignored": (
        "carried[k] = state_in ? state_in[(b * dim + d) * width + k] : 0.0;",
        "carried[k] = 0.0;"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle_build.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for '{name}' not unique in the oracle source"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle_build.compile_oracle(str(src), str(tmp_path / "libmutant.so"))
    mutant = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError as e:
            failed.append((pin.__name__, str(e)[:80]))
    assert failed, f"no pin caught the planted mistake '{name}'"
