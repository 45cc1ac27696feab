"""GPU parity of the backward scan (ssm_scan_bwd through the C ABI) against
the fp64 CPU oracle's backward pass on the same seeded inputs.

Tolerance, per gradient tensor: max abs error <= tol * max|oracle| with
tol = 1e-4 for fp32 I/O and 2e-2 for bf16 I/O. The fp32 bound is looser than
the forward's 1e-5: each gradient combines states recomputed in fp32 (a
forward pass over the whole sequence to the checkpoints, then up to 8 tokens
from a checkpoint) with an adjoint carried back over the whole sequence,
through the hardware exp2 (about 1 ulp) and fp32 accumulation, and dA, dB
and dC add thousands of such terms. bf16 I/O keeps the forward's 2e-2 (dx, ddelta, dz
are rounded to bf16 on output).
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import selective_state_space_40_amd as ms
import ssm_workloads as W
from parity_util import assert_close, sample_channels

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL_BWD = {"f32": 1e-4, "bf16": 2e-2}
KEYS = ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0", "ddelta_bias")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ms.load_library()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(batch, seqlen, dim, dstate, io, seed, h0=True, D=True, z=True, softplus=False):
    w = dataclasses.replace(W.WORKLOADS["mamba130m_layer"], io=io, dstate=dstate,
                            h0="normal" if h0 else "zero")
    inp = W.generate_scan(w, device=DEV, batch=batch, seqlen=seqlen, dim=dim, seed=seed,
                          raw_delta=softplus)
    if not D:
        inp["D"] = None
    if not z:
        inp["z"] = None
    g = torch.Generator(device=DEV).manual_seed(seed + 7)
    dy = torch.randn(batch, seqlen, dim, generator=g, device=DEV).to(inp["x"].dtype)
    dhL = torch.randn(batch, dim, dstate, generator=g, device=DEV)
    return inp, dy, dhL


def _compare(orc, inp, dy, dhL, io, what, keys=KEYS, halves=ms.HALVES_AUTO, chunk_len=0):
    sp = inp.get("delta_bias") is not None
    got = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                      inp.get("z"), inp.get("h0"), dy=dy, dhL=dhL,
                      delta_bias=inp.get("delta_bias"), delta_softplus=sp, halves=halves,
                      chunk_len=chunk_len)
    torch.cuda.synchronize()
    want = orc.scan_bwd(**inp, dy=dy, dhL=dhL, delta_softplus=sp)
    for k in keys:
        if want[k] is None:
            assert got[k] is None, f"{what}: {k} should be absent"
            continue
        assert_close(got[k], want[k], TOL_BWD[io], f"{what} {k}")
    return got


CASES = [
    # (batch, seqlen, dim, dstate, io)
    (1, 1, 1, 1, "f32"), (2, 7, 3, 4, "f32"), (1, 8, 64, 16, "f32"), (2, 31, 65, 16, "f32"),
    (1, 32, 64, 8, "bf16"), (2, 33, 130, 16, "f32"), (1, 64, 70, 5, "f32"),
    (2, 100, 64, 12, "bf16"), (1, 257, 96, 16, "f32"), (3, 45, 200, 3, "f32"),
    (2, 129, 128, 16, "bf16"), (1, 77, 33, 2, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_shapes(orc, case):
    batch, seqlen, dim, dstate, io = case
    inp, dy, dhL = _inputs(*case, seed=sum(case[:4]))
    _say(f"case bwd {case}")
    _compare(orc, inp, dy, dhL, io, f"bwd {case}")


HALF_CASES = [
    # (batch, seqlen, dim, dstate, io): dim 70 leaves the second half of its
    # last group wholly past the last channel, dim 100 a half with 4 real
    # channels; N = 13 pads the last split's states
    (2, 31, 65, 16, "f32"), (3, 45, 100, 16, "f32"), (2, 50, 70, 13, "f32"),
    (2, 129, 128, 16, "bf16"), (1, 257, 96, 14, "f32"),
]


@pytest.mark.parametrize("case", HALF_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_half_groups(orc, case):
    # every split group count: none, one, half of them, all
    batch, seqlen, dim, dstate, io = case
    inp, dy, dhL = _inputs(*case, seed=sum(case[:4]) + 1)
    G = batch * ((dim + 63) // 64)
    for halves in sorted({ms.HALVES_NONE, 1, max(1, G // 2), G}):
        _say(f"case bwd halves={halves} of {G} groups {case}")
        _compare(orc, inp, dy, dhL, io, f"bwd halves={halves} {case}", halves=halves)


def test_bwd_half_groups_options_and_softplus(orc):
    for h0, D, z, use_dhL in ((False, True, True, True), (True, False, False, False)):
        inp, dy, dhL = _inputs(2, 70, 80, 16, "f32", seed=5, h0=h0, D=D, z=z)
        _say(f"case bwd halves=all h0={h0} D={D} z={z} dhL={use_dhL}")
        _compare(orc, inp, dy, dhL if use_dhL else None, "f32",
                 f"bwd halves h0={h0} D={D} z={z} dhL={use_dhL}", halves=4)
    for io in ("f32", "bf16"):
        inp, dy, dhL = _inputs(2, 90, 100, 16, io, seed=6, softplus=True)
        _say(f"case bwd halves softplus {io}")
        _compare(orc, inp, dy, dhL, io, f"bwd halves softplus {io}", halves=3)


def test_bwd_half_groups_bitwise_run_to_run():
    inp, dy, dhL = _inputs(2, 60, 150, 16, "bf16", seed=8)

    def run():
        g = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                        inp["h0"], dy=dy, dhL=dhL, halves=4)
        torch.cuda.synchronize()
        return g
    a, b = run(), run()
    for k in KEYS:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def test_bwd_optional_inputs(orc):
    for h0, D, z, use_dhL in ((False, True, True, True), (True, False, True, False),
                              (True, True, False, True), (False, False, False, False)):
        inp, dy, dhL = _inputs(2, 70, 80, 16, "f32", seed=3, h0=h0, D=D, z=z)
        _say(f"case bwd h0={h0} D={D} z={z} dhL={use_dhL}")
        _compare(orc, inp, dy, dhL if use_dhL else None, "f32",
                 f"bwd h0={h0} D={D} z={z} dhL={use_dhL}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_fused_softplus(orc, io):
    for dstate in (16, 5):
        inp, dy, dhL = _inputs(2, 90, 100, dstate, io, seed=dstate, softplus=True)
        _say(f"case bwd softplus N={dstate} {io}")
        _compare(orc, inp, dy, dhL, io, f"bwd softplus N={dstate} {io}")


def test_bwd_full_size_sampled(orc):
    # the Mamba-2.8B layer shape: per-channel gradients on sampled channels
    # over all rows, and dB/dC (sums over all channels) on every row
    w = W.WORKLOADS["mamba28b_layer"]
    inp = W.generate_scan(w, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(99)
    dy = torch.randn(w.batch, w.seqlen, w.dim, generator=g, device=DEV).to(torch.bfloat16)
    _say(f"case bwd {w.name} full size")
    got = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                      inp["h0"], dy=dy)
    torch.cuda.synchronize()
    idx = sample_channels(w.dim, count=12, seed=w.seed)
    ix = torch.as_tensor(idx, device=DEV)
    sub = dict(x=inp["x"].index_select(2, ix), delta=inp["delta"].index_select(2, ix),
               A=inp["A"].index_select(0, ix), B=inp["B"], C=inp["C"],
               D=inp["D"].index_select(0, ix), z=inp["z"].index_select(2, ix), h0=None)
    _say(f"case bwd {w.name}: oracle on {len(idx)} channels")
    want = orc.scan_bwd(**sub, dy=dy.index_select(2, ix))
    for k, dim_axis in (("dx", 2), ("ddelta", 2), ("dz", 2)):
        assert_close(got[k].index_select(dim_axis, ix), want[k], TOL_BWD["bf16"], f"full {k}")
    assert_close(got["dA"].index_select(0, ix), want["dA"], TOL_BWD["bf16"], "full dA")
    assert_close(got["dD"].index_select(0, ix), want["dD"], TOL_BWD["bf16"], "full dD")
    assert_close(got["dh0"].index_select(1, ix), want["dh0"], TOL_BWD["bf16"], "full dh0")
    # dB and dC sum over all 5,120 channels: the oracle over every row and
    # channel, one row at a time
    for b in range(w.batch):
        _say(f"case bwd {w.name}: oracle on batch row {b}, all channels")
        row = {k: (v[b:b + 1] if k in ("x", "delta", "B", "C", "z") else v)
               for k, v in inp.items()}
        want_b = orc.scan_bwd(**row, dy=dy[b:b + 1])
        assert_close(got["dB"][b:b + 1], want_b["dB"], TOL_BWD["bf16"], f"full dB (row {b})")
        assert_close(got["dC"][b:b + 1], want_b["dC"], TOL_BWD["bf16"], f"full dC (row {b})")
    _check_projections(inp, dy, got, range(0, w.seqlen, 1), "full")


def _check_projections(inp, dy, got, tokens, what):
    """Two identities that hold at any size, for the sums over channels:
    y = silu(z) (C.h + D x) gives sum_n C[t,n] dC[t,n] = sum_d dy (y - silu(z) D x),
    and dx = delta sum_n lam B + D dy silu(z) gives
    sum_n B[t,n] dB[t,n] = sum_d x (dx - D dy silu(z)) (lam: the adjoint of the
    state after token t). y comes from the forward scan of the same inputs
    (checked against the oracle elsewhere); every side in fp64; the bound is
    relative to the sum of the magnitudes of each side's terms."""
    y, _ = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                       inp["z"], inp["h0"])
    torch.cuda.synchronize()
    t = torch.as_tensor(list(tokens), device=DEV)
    f = lambda v: v.index_select(1, t).double()
    x, z, dyt, yt, dx = f(inp["x"]), f(inp["z"]), f(dy), f(y), f(got["dx"])
    Bt, Ct, dB, dC = f(inp["B"]), f(inp["C"]), f(got["dB"]), f(got["dC"])
    g = z * torch.sigmoid(z)
    Dx = inp["D"].double() * x
    for lhs_terms, rhs_terms, name in (
            (Ct * dC, dyt * (yt - g * Dx), "C.dC"),
            (Bt * dB, x * (dx - inp["D"].double() * dyt * g), "B.dB")):
        lhs, rhs = lhs_terms.sum(-1), rhs_terms.sum(-1)
        scale = lhs_terms.abs().sum(-1) + rhs_terms.abs().sum(-1)
        err = ((lhs - rhs).abs() / scale.clamp_min(1e-30)).max().item()
        assert err <= TOL_BWD["bf16"], f"{what}: {name} identity off by {err:.3e} (relative)"


def test_bwd_empty_and_deterministic(orc):
    inp, dy, dhL = _inputs(2, 0, 40, 16, "f32", seed=5)
    got = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                      inp["h0"], dy=dy, dhL=dhL)
    torch.cuda.synchronize()
    assert torch.count_nonzero(got["dA"]) == 0 and torch.count_nonzero(got["dD"]) == 0
    assert torch.equal(got["dh0"], dhL)
    inp, dy, dhL = _inputs(2, 300, 130, 16, "bf16", seed=6)
    a = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], dy=dy, dhL=dhL)
    b = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], dy=dy, dhL=dhL)
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), f"{k} not reproducible"


@pytest.mark.parametrize("halves", [ms.HALVES_AUTO, ms.HALVES_NONE], ids=["halves", "whole"])
def test_bwd_nan_propagates_like_the_oracle(orc, halves):
    # a NaN in one x: every gradient is NaN exactly where the oracle's is
    # (d delta, dz and dC from that token on, dB at that token, dA and dD of
    # that channel), finite entries within tolerance; dx and dh0 stay finite
    inp, dy, dhL = _inputs(2, 37, 70, 16, "f32", seed=41)
    t, d = 20, 5
    inp["x"][1, t, d] = float("nan")
    _say(f"case backward with a NaN input, halves={halves}")
    got = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                      inp["h0"], dy=dy, dhL=dhL, halves=halves)
    torch.cuda.synchronize()
    want = orc.scan_bwd(**inp, dy=dy, dhL=dhL)
    for k in KEYS:
        if want[k] is None:
            continue
        g = got[k].double().cpu().numpy()
        w = np.asarray(want[k], dtype=np.float64)
        assert np.array_equal(np.isnan(g), np.isnan(w)), f"{k}: NaN positions differ"
        fin = np.isfinite(w)
        assert np.all(np.isfinite(g[fin])), f"{k}: non-finite where the oracle is finite"
        scale = float(np.max(np.abs(w[fin]))) if fin.any() else 0.0
        err = float(np.max(np.abs(g[fin] - w[fin]))) if fin.any() else 0.0
        assert err <= TOL_BWD["f32"] * scale, f"{k}: max abs error {err:.3e} vs {scale:.3e}"
    wnan = {k: np.isnan(np.asarray(want[k], dtype=np.float64)) for k in KEYS if want[k] is not None}
    assert wnan["ddelta"][1, t:, d].all() and not wnan["ddelta"][1, :t, d].any()
    assert wnan["dz"][1, t:, d].all() and wnan["dC"][1, t:].all() and wnan["dB"][1, t].all()
    assert wnan["dA"][d].all() and wnan["dD"][d] and not wnan["dx"].any() and not wnan["dh0"].any()


# ---------------------------------------------------------------------------
# sequences cut into chunks: state and adjoint summaries folded across chunks

CHUNK_CASES = [
    # (batch, seqlen, dim, dstate, io, chunk_len)
    (1, 257, 70, 16, "f32", 64),     # ragged last chunk and tile, 5 chunks
    (2, 300, 130, 12, "bf16", 72),   # chunk not a power of two, 3 waves
    (1, 200, 64, 5, "f32", 64),      # 2 waves
    (1, 129, 33, 2, "f32", 8),       # one tile per chunk, 17 chunks
    (3, 100, 20, 4, "f32", 24),
    (2, 64, 64, 16, "f32", 64),      # chunk_len == seqlen: one chunk
    (1, 300, 96, 13, "bf16", 48),    # 4 waves, the last with padding states
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_chunked(orc, case):
    batch, seqlen, dim, dstate, io, cl = case
    inp, dy, dhL = _inputs(batch, seqlen, dim, dstate, io, seed=seqlen + dim + cl)
    _say(f"case backward chunked {case}")
    _compare(orc, inp, dy, dhL, io, f"chunked {case}", chunk_len=cl)


def test_bwd_chunked_options_and_softplus(orc):
    inp, dy, dhL = _inputs(2, 150, 96, 16, "f32", seed=61, h0=False, D=False, z=False)
    _say("case backward chunked without D, z, h0, dhL")
    _compare(orc, inp, dy, None, "f32", "chunked bare", chunk_len=40)
    inp, dy, dhL = _inputs(2, 150, 96, 16, "bf16", seed=62, softplus=True)
    _say("case backward chunked with fused softplus")
    _compare(orc, inp, dy, dhL, "bf16", "chunked softplus", chunk_len=48)


def test_bwd_chunked_agrees_with_one_chunk():
    inp, dy, dhL = _inputs(1, 500, 192, 16, "f32", seed=63)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["h0"])
    one = ms.scan_bwd(*args, dy=dy, dhL=dhL, chunk_len=0, halves=ms.HALVES_NONE)
    cut = ms.scan_bwd(*args, dy=dy, dhL=dhL, chunk_len=96)
    again = ms.scan_bwd(*args, dy=dy, dhL=dhL, chunk_len=96)
    torch.cuda.synchronize()
    for k in KEYS:
        if one[k] is None:
            continue
        assert_close(cut[k], one[k], 2e-5, f"chunked vs one chunk {k}")
        assert torch.equal(cut[k], again[k]), f"chunked run to run {k}"


def test_bwd_automatic_plan_cuts_small_batch(orc):
    # one row of 130 channels: 3 groups cannot fill the chip, so the plan
    # cuts the sequence; the result still matches the oracle
    plan = ms.resolve_bwd_plan(1, 2048, 130, 16, torch.float32)
    assert 64 <= plan.chunk_len < 2048 and plan.chunk_len % 8 == 0 and plan.halves == 0
    big = ms.resolve_bwd_plan(8, 2048, 5120, 16, torch.bfloat16)
    assert big.chunk_len == 2048          # the Mamba-2.8B layer stays whole
    inp, dy, dhL = _inputs(1, 2048, 130, 16, "f32", seed=64)
    _say(f"case backward automatic plan, chunks of {plan.chunk_len}")
    _compare(orc, inp, dy, dhL, "f32", "automatic chunks")


def test_bwd_chunks_and_halves_together_rejected():
    inp, dy, dhL = _inputs(1, 128, 64, 16, "f32", seed=65)
    with pytest.raises(ms.MambaScanError):
        ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], dy=dy, dhL=dhL, chunk_len=64, halves=1)


def test_bwd_million_length_sampled(orc):
    # one row of 2048 channels over 2^20 tokens: the plan cuts the sequence
    # into chunks; per-channel gradients on sampled channels against the
    # oracle over the whole sequence; dB and dC (sums over every channel)
    # through two identities that hold at any size (_check_projections)
    w = W.WORKLOADS["million_length"]
    plan = ms.resolve_bwd_plan(w.batch, w.seqlen, w.dim, w.dstate, torch.bfloat16)
    assert plan.chunk_len < w.seqlen
    inp = W.generate_scan(w, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(98)
    dy = torch.randn(w.batch, w.seqlen, w.dim, generator=g, device=DEV).to(torch.bfloat16)
    _say(f"case bwd {w.name} full size, chunks of {plan.chunk_len}")
    got = ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                      inp["h0"], dy=dy)
    torch.cuda.synchronize()
    idx = sample_channels(w.dim, count=6, seed=w.seed)
    ix = torch.as_tensor(idx, device=DEV)
    sub = dict(x=inp["x"].index_select(2, ix), delta=inp["delta"].index_select(2, ix),
               A=inp["A"].index_select(0, ix), B=inp["B"], C=inp["C"],
               D=inp["D"].index_select(0, ix), z=inp["z"].index_select(2, ix), h0=None)
    _say(f"case bwd {w.name}: oracle on {len(idx)} channels")
    want = orc.scan_bwd(**sub, dy=dy.index_select(2, ix))
    for k in ("dx", "ddelta", "dz"):
        assert_close(got[k].index_select(2, ix), want[k], TOL_BWD["bf16"], f"million {k}")
    assert_close(got["dA"].index_select(0, ix), want["dA"], TOL_BWD["bf16"], "million dA")
    assert_close(got["dD"].index_select(0, ix), want["dD"], TOL_BWD["bf16"], "million dD")
    assert_close(got["dh0"].index_select(1, ix), want["dh0"], TOL_BWD["bf16"], "million dh0")
    # dB and dC (sums over all 2,048 channels) through the identities, on
    # every 64th token and on the tokens around every chunk boundary
    _say(f"case bwd {w.name}: dB/dC identities")
    toks = set(range(0, w.seqlen, 64))
    for c in range(plan.chunk_len, w.seqlen, plan.chunk_len):
        toks.update(range(max(0, c - 8), min(w.seqlen, c + 8)))
    _check_projections(inp, dy, got, sorted(toks), "million")
