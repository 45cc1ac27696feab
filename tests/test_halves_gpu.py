"""GPU: single-chunk scans with half channel groups, through the C ABI.

The plan can run the last channel groups (64 channels of one batch row) as
two halves of 32 channels whose states spread over 8 lanes each, so that a
launch puts the same work on every compute unit. The outputs are checked
against the fp64 oracle (parity_util.TOL) with every group split, some
split and none split, on ragged channel counts (a half partly past the
last channel, a second half wholly past it), ragged and very short
sequences, N = 8 and 16, both I/O dtypes, the fused delta activation, the
optional inputs and an aliased state. The automatic plan of the
Mamba-2.8B layer shape splits exactly the groups one round of the chip
leaves over.
"""
import sys

import pytest
import torch

import selective_state_space_40_amd as ms
import ssm_workloads as W
from parity_util import TOL, assert_close

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


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


def _inputs(batch, seqlen, dim, dstate, io, seed):
    """x, z, B, C, h0, D ~ N(0,1); delta = softplus(N(0,1) - 1);
    A = -exp(U(-1,1))."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = W.io_torch_dtype(io)

    def n(*s):
        return torch.randn(*s, generator=g)
    inp = dict(
        x=n(batch, seqlen, dim).to(dt),
        delta=torch.nn.functional.softplus(n(batch, seqlen, dim) - 1.0).to(dt),
        A=-torch.exp(torch.rand(dim, dstate, generator=g) * 2 - 1),
        B=n(batch, seqlen, dstate).to(dt), C=n(batch, seqlen, dstate).to(dt),
        D=n(dim), z=n(batch, seqlen, dim).to(dt), h0=n(batch, dim, dstate))
    return {k: v.to(DEV) for k, v in inp.items()}


def _run(inp, halves, **kw):
    L = inp["x"].shape[1]
    y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                        inp.get("z"), inp.get("h0"), chunk_len=max(L, 1), state_split=4,
                        halves=halves, **kw)
    torch.cuda.synchronize()
    return y, hL


# (batch, seqlen, dim, dstate, io): ragged tiles and channel groups; dim 70
# leaves the second half of its last group wholly past the last channel,
# dim 100 a half with 4 real channels
CASES = [
    (2, 203, 100, 16, "f32"),
    (3, 77, 70, 16, "bf16"),
    (1, 5, 64, 16, "f32"),
    (2, 1, 130, 16, "f32"),
    (2, 150, 96, 8, "f32"),
    (1, 64, 256, 8, "bf16"),
]


def _groups(case):
    batch, _, dim, _, _ = case
    return batch * ((dim + 63) // 64)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_halves_match_oracle(orc, case):
    batch, seqlen, dim, dstate, io = case
    inp = _inputs(batch, seqlen, dim, dstate, io, seed=seqlen * 7 + dim + dstate)
    yo, ho = orc.scan_fwd(**inp)
    G = _groups(case)
    for halves in sorted({G, max(1, G // 2), 1, ms.HALVES_NONE}):
        _say(f"case halves={halves} of {G} groups, shape {case}")
        y, hL = _run(inp, halves)
        assert_close(y, yo, TOL[io], f"halves {halves} {case} y")
        assert_close(hL, ho, TOL[io], f"halves {halves} {case} hL")


def test_halves_agree_with_whole_groups():
    # the same scan with every group whole and every group halved: only the
    # order of the readout sums differs (8 partials against 4)
    inp = _inputs(2, 500, 192, 16, "f32", seed=31)
    y1, h1 = _run(inp, ms.HALVES_NONE)
    y2, h2 = _run(inp, 6)
    assert_close(y2, y1, 2e-6, "halved vs whole y")
    assert torch.equal(h1, h2) or float((h1 - h2).abs().max()) <= 1e-6 * float(h1.abs().max())


def test_halves_with_fused_softplus_and_without_options(orc):
    inp = _inputs(2, 120, 160, 16, "bf16", seed=32)
    raw = (inp["delta"].float() - 0.5).to(torch.bfloat16)
    bias = torch.randn(160, generator=torch.Generator().manual_seed(4)).to(DEV) * 0.3
    inp["delta"] = raw
    inp["delta_bias"] = bias
    _say("case halves with delta bias + softplus")
    y, hL = _run(inp, 6, delta_bias=bias, delta_softplus=True)
    yo, ho = orc.scan_fwd(**inp, delta_softplus=True)
    assert_close(y, yo, TOL["bf16"], "halves softplus y")
    assert_close(hL, ho, TOL["bf16"], "halves softplus hL")
    bare = {k: v for k, v in inp.items() if k not in ("D", "z", "h0", "delta_bias")}
    bare["delta"] = torch.nn.functional.softplus(raw.float() + bias).to(torch.bfloat16)
    _say("case halves without D, z, h0, hL")
    y, hL = ms.scan_fwd(bare["x"], bare["delta"], bare["A"], bare["B"], bare["C"], None, None,
                        None, chunk_len=120, state_split=4, halves=6, return_state=False)
    torch.cuda.synchronize()
    assert hL is None
    yo, _ = orc.scan_fwd(**bare)
    assert_close(y, yo, TOL["bf16"], "halves bare y")


def test_halves_state_aliasing(orc):
    inp = _inputs(2, 90, 128, 16, "f32", seed=33)
    yo, ho = orc.scan_fwd(**inp)
    h = inp["h0"]
    _say("case halves, hL aliases h0")
    y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                        h, state_out=h, chunk_len=90, state_split=4, halves=3)
    torch.cuda.synchronize()
    assert hL.data_ptr() == h.data_ptr()
    assert_close(y, yo, TOL["f32"], "aliased y")
    assert_close(h, ho, TOL["f32"], "aliased state")


def test_halves_bitwise_run_to_run():
    inp = _inputs(2, 300, 200, 16, "bf16", seed=34)
    y1, h1 = _run(inp, 5)
    y2, h2 = _run(inp, 5)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_automatic_plan_splits_the_surplus_groups():
    # 8 rows x 80 groups = 640 groups; with C compute units the plan splits
    # the 640 mod C groups left over by whole rounds when they are at most C/2
    cu = torch.cuda.get_device_properties(DEV).multi_processor_count
    plan = ms.resolve_plan(8, 2048, 5120, 16, torch.bfloat16)
    surplus = 640 % cu
    want = surplus if 0 < surplus and 2 * surplus <= cu else 0
    assert (plan.chunk_len, plan.state_split, plan.halves) == (2048, 4, want)
