"""GPU: the repaired carry of a chunked scan, through the C ABI.

Every chunk runs once from a zero state (chunk 0 from h0) and writes y; the
fold of the chunk summaries gives each chunk's entering state and hL; each
later chunk is then rerun from its entering state only while exp(A * sum of
delta since the chunk start) exceeds 2^-32 for some state of its 64-channel
group. The outputs are checked against the fp64 oracle (parity_util.TOL),
against the summary-pass carry on the same inputs, and where the entering
state never decays (an A of 0, delta near 0, a NaN) against the summary-pass
carry bit for bit: the rerun then covers the whole chunk with the same
arithmetic.
"""
import sys

import pytest
import torch

import selective_state_space_40_amd as ms
import ssm_workloads as W
from parity_util import TOL, assert_close

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPAIR, RERUN = ms.CARRY_REPAIR, ms.CARRY_RERUN


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


def _inputs(batch, seqlen, dim, dstate, io, seed, delta_shift=-1.0):
    """x, z, B, C ~ N(0,1); delta = softplus(N(0,1) + delta_shift);
    A = -exp(U(-1,1)); D ~ N(0,1); h0 ~ N(0,1)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = W.io_torch_dtype(io)

    def n(*s):
        return torch.randn(*s, generator=g)
    inp = dict(
        x=n(batch, seqlen, dim).to(dt),
        delta=torch.nn.functional.softplus(n(batch, seqlen, dim) + delta_shift).to(dt),
        A=-torch.exp(torch.rand(dim, dstate, generator=g) * 2 - 1),
        B=n(batch, seqlen, dstate).to(dt), C=n(batch, seqlen, dstate).to(dt),
        D=n(dim), z=n(batch, seqlen, dim).to(dt), h0=n(batch, dim, dstate))
    return {k: v.to(DEV) for k, v in inp.items()}


def _run(inp, **kw):
    y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                        inp["z"], inp["h0"], **kw)
    torch.cuda.synchronize()
    return y, hL


# (batch, seqlen, dim, dstate, io, chunk_len, state_split): ragged last
# chunks, tiles and channel groups; heads that stop inside every chunk
# (delta ~ softplus(N(0,1) - 1) forgets the entering state within ~150
# tokens) and, with 64-token chunks, reruns that cover whole chunks
CASES = [
    (2, 3000, 72, 16, "f32", 512, 4),
    (2, 3000, 72, 16, "f32", 512, 1),
    (2, 2100, 100, 8, "bf16", 700, 2),
    (1, 1500, 64, 5, "f32", 300, 1),
    (2, 4500, 40, 4, "f32", 1000, 4),
    (3, 999, 130, 16, "bf16", 64, 8),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_repaired_carry_matches_oracle(orc, case):
    batch, seqlen, dim, dstate, io, chunk_len, split = case
    inp = _inputs(batch, seqlen, dim, dstate, io, seed=seqlen + dim + dstate)
    _say(f"case repaired carry {case}")
    y, hL = _run(inp, chunk_len=chunk_len, state_split=split, carry=REPAIR)
    yo, ho = orc.scan_fwd(**inp)
    assert_close(y, yo, TOL[io], f"repaired {case} y")
    assert_close(hL, ho, TOL[io], f"repaired {case} hL")


def test_repaired_carry_agrees_with_rerun():
    # fp32 I/O, ordinary magnitudes: the dropped share of the entering state
    # (< 2^-32 of its readout) is far below fp32 rounding, so the kept
    # zero-start outputs agree with the rerun ones (in practice bit for bit:
    # once the difference of the two states rounds away they coincide)
    inp = _inputs(2, 3000, 72, 16, "f32", seed=21)
    _say("case repaired vs rerun carry, fast decay")
    y1, h1 = _run(inp, chunk_len=512, state_split=4, carry=REPAIR)
    y2, h2 = _run(inp, chunk_len=512, state_split=4, carry=RERUN)
    assert_close(y1, y2, 1e-6, "repaired vs rerun y")
    assert_close(h1, h2, 1e-6, "repaired vs rerun hL")


def _huge_entering_state(orc, dim, undecayed=None):
    """One batch row, two 512-token chunks, fp32. h0 ~ 1e20 * N(0,1) and a
    delta of 1e-7 over chunk 0 carry an enormous state into chunk 1, whose
    delta ~ softplus(N(0,1) - 1) forgets it within ~150 tokens: there the
    share the repaired carry drops, up to 2^-32 of the entering state's
    readout, is far above rounding and shows. Returns the inputs, the state
    entering chunk 1 (fp64 oracle) and the outputs of both carries."""
    inp = _inputs(1, 1024, dim, 16, "f32", seed=28)
    inp["h0"] = inp["h0"] * 1e20
    inp["delta"][:, :512] = 1e-7
    if undecayed is not None:
        inp["A"][undecayed] = 0.0
    head = {k: (v[:, :512] if k in ("x", "delta", "B", "C", "z") else v) for k, v in inp.items()}
    _, h_in = orc.scan_fwd(**head)
    y1, _ = _run(inp, chunk_len=512, state_split=4, carry=REPAIR)
    y2, _ = _run(inp, chunk_len=512, state_split=4, carry=RERUN)
    return inp, h_in, y1.double().cpu(), y2.double().cpu()


def test_repaired_carry_keeps_its_bound(orc):
    # where the entering state is huge the head rerun visibly stops early,
    # and every kept output stays within the stated bound of the rerun one:
    # |y_repair - y_rerun| <= |silu(z)| * 2^-32 * sum_n |C[n] h_in[n]|
    # (plus fp32 rounding of the rerun output itself)
    _say("case repaired carry bound, huge entering state")
    inp, h_in, y1, y2 = _huge_entering_state(orc, 64)
    z = inp["z"][0, 512:].double().cpu()
    C = inp["C"][0, 512:].double().cpu()                       # (512, N)
    hin = torch.as_tensor(h_in[0]).double()                    # (dim, N)
    readout = C.abs() @ hin.abs().T                            # (512, dim)
    bound = (z * torch.sigmoid(z)).abs() * readout * 2.0 ** -32
    diff = (y1[0, 512:] - y2[0, 512:]).abs()
    assert torch.all(diff <= bound * 1.001 + 1e-5 * y2[0, 512:].abs() + 1e-30)
    # the first tokens of chunk 1 are rerun (the state still counts there) ...
    assert torch.allclose(y1[0, 512:560], y2[0, 512:560], rtol=1e-5, atol=0)
    # ... and the rerun stopped before the chunk's end: past the stop the
    # dropped share (up to ~1e10 here) shows until it decays under rounding
    assert not torch.equal(y1[0, 512:], y2[0, 512:])


def test_undecayed_group_reruns_whole_chunks(orc):
    # A = 0 for one state of channel 3 (outside the A < 0 precondition, so its
    # entering state never fades): channel group 0 (channels 0..63) reruns
    # every chunk to its end with the rerun form's arithmetic, bit for bit,
    # while group 1 (channels 64..99) stops early and keeps its zero-start tail
    _say("case repaired carry with an undecayed state")
    _, _, y1, y2 = _huge_entering_state(orc, 100, undecayed=(3, 5))
    assert torch.equal(y1[:, :, :64], y2[:, :, :64])
    assert not torch.equal(y1[:, 512:, 64:], y2[:, 512:, 64:])


def test_slow_decay_reruns_whole_chunks(orc):
    # delta ~ softplus(N(0,1) - 9) ~ 1e-4: the entering state never fades
    # within a chunk, so every chunk is rerun whole, bit for bit as the rerun form
    inp = _inputs(2, 1200, 70, 16, "bf16", seed=23, delta_shift=-9.0)
    _say("case repaired carry, slow decay")
    y1, h1 = _run(inp, chunk_len=300, state_split=4, carry=REPAIR)
    y2, _ = _run(inp, chunk_len=300, state_split=4, carry=RERUN)
    assert torch.equal(y1, y2)
    yo, ho = orc.scan_fwd(**inp)
    assert_close(y1, yo, TOL["bf16"], "slow decay y")
    assert_close(h1, ho, TOL["bf16"], "slow decay hL")


def test_repaired_carry_propagates_nan():
    # a NaN input in chunk 0 makes every later entering state of its channel
    # NaN; non-finite entering states are rerun whole, so the NaN reaches
    # every later output of that channel, as in the rerun form
    inp = _inputs(1, 2000, 64, 16, "f32", seed=24)
    inp["x"][0, 100, 5] = float("nan")
    _say("case repaired carry, NaN in the first chunk")
    y, hL = _run(inp, chunk_len=500, state_split=4, carry=REPAIR)
    assert torch.isnan(y[0, 100:, 5]).all()
    assert torch.isnan(hL[0, 5]).all()
    assert torch.isfinite(y[0, :100]).all() and torch.isfinite(y[0, :, 6]).all()


def test_repaired_carry_state_aliasing(orc):
    # hL may alias h0: pass 1 reads h0 before the fold writes hL
    inp = _inputs(2, 1100, 90, 16, "f32", seed=25)
    yo, ho = orc.scan_fwd(**inp)
    h = inp["h0"]
    _say("case repaired carry, hL aliases h0")
    y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                        inp["z"], h, state_out=h, chunk_len=256, carry=REPAIR)
    torch.cuda.synchronize()
    assert hL.data_ptr() == h.data_ptr()
    assert_close(y, yo, TOL["f32"], "aliased y")
    assert_close(h, ho, TOL["f32"], "aliased state")


def test_repaired_carry_without_state_or_options(orc):
    # no h0, no hL, no D, no z: the fold skips the last chunk's step
    inp = _inputs(2, 1300, 80, 16, "f32", seed=26)
    for k in ("h0", "D", "z"):
        inp[k] = None
    _say("case repaired carry without optional inputs")
    y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], None, None, None,
                        chunk_len=256, carry=REPAIR, return_state=False)
    torch.cuda.synchronize()
    assert hL is None
    yo, _ = orc.scan_fwd(**inp)
    assert_close(y, yo, TOL["f32"], "repaired y without optional inputs")


def test_repaired_carry_with_fused_softplus(orc):
    inp = _inputs(2, 1600, 100, 16, "bf16", seed=27)
    raw = inp["delta"].float()
    bias = torch.randn(100, generator=torch.Generator().manual_seed(3)).to(DEV) * 0.5
    # raw delta whose activation softplus(raw + bias) is the decay step
    inp["delta"] = (raw - 1.0).to(torch.bfloat16)
    inp["delta_bias"] = bias
    _say("case repaired carry with delta bias + softplus")
    y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                        inp["z"], inp["h0"], delta_bias=bias, delta_softplus=True,
                        chunk_len=320, carry=REPAIR)
    torch.cuda.synchronize()
    yo, ho = orc.scan_fwd(**inp, delta_softplus=True)
    assert_close(y, yo, TOL["bf16"], "repaired softplus y")
    assert_close(hL, ho, TOL["bf16"], "repaired softplus hL")


def _splits(dstate):
    # the splits the kernels are built for at this state size (besides 1)
    return [1] + [s for s in (2, 4, 8) if dstate in (4, 8, 16) and dstate % s == 0]


@pytest.mark.parametrize("dstate", list(range(1, ms.MAX_DSTATE + 1)))
def test_repaired_carry_every_state_size(orc, dstate):
    # every compiled state size and split of the local and fix-up kernels:
    # 5 chunks of 160 tokens (the last ragged), 70 channels (a ragged group)
    inp = _inputs(1, 700, 70, dstate, "f32", seed=40 + dstate)
    yo, ho = orc.scan_fwd(**inp)
    for split in _splits(dstate):
        _say(f"case repaired carry N={dstate} split={split}")
        y, hL = _run(inp, chunk_len=160, state_split=split, carry=REPAIR)
        assert_close(y, yo, TOL["f32"], f"repaired N={dstate} split={split} y")
        assert_close(hL, ho, TOL["f32"], f"repaired N={dstate} split={split} hL")
