"""GPU parity: the HIP scan and decode kernels, called through the C ABI,
against the fp64 CPU oracle on the same seeded inputs.

Tolerance (parity_util.TOL): max abs error <= 1e-5 * max|oracle| for fp32
I/O and <= 2e-2 * max|oracle| for bf16 I/O with fp32 state, on y and on the
final state. Full-size workloads run in the same launch configuration the
benchmark times (automatic chunk plan) and are compared on sampled channels
over every batch row and every token; small cases are compared everywhere.
"""
import sys

import numpy as np
import pytest
import torch

import selective_state_space_40_amd as ms
import ssm_workloads as W
from parity_util import TOL, assert_close, oracle_on_channels, sample_channels

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


def _gen(w, **kw):
    return {k: (v.to(DEV) if v is not None else None) for k, v in W.generate_scan(w, **kw).items()}


def _run(inp, **kw):
    y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                        inp.get("z"), inp.get("h0"), **kw)
    torch.cuda.synchronize()
    return y, hL


def _full_compare(orc, inp, y, hL, tol, what):
    yo, ho = orc.scan_fwd(**inp)
    assert_close(y, yo, tol, f"{what} y")
    assert_close(hL, ho, tol, f"{what} hL")


# ---------------------------------------------------------------------------
# the five workloads


def test_tiny_f32(orc):
    w = W.WORKLOADS["tiny_f32"]
    inp = _gen(w)
    _say("case tiny_f32 B=1 L=64 D=16 N=4 fp32")
    y, hL = _run(inp)
    _full_compare(orc, inp, y, hL, TOL["f32"], "tiny_f32")


@pytest.mark.parametrize("name", ["mamba130m_layer", "mamba28b_layer"])
def test_layer_scan_full_size_sampled(orc, name):
    w = W.WORKLOADS[name]
    inp = W.generate_scan(w, device=DEV)
    _say(f"case {name} B={w.batch} L={w.seqlen} D={w.dim} N={w.dstate} bf16, automatic plan")
    y, hL = _run(inp)
    idx = sample_channels(w.dim, seed=w.seed)
    yo, ho = oracle_on_channels(orc, inp, idx)
    ix = torch.as_tensor(idx, device=DEV)
    assert_close(y.index_select(2, ix), yo, TOL["bf16"], f"{name} y (sampled channels)")
    assert_close(hL.index_select(1, ix), ho, TOL["bf16"], f"{name} hL (sampled channels)")


def test_layer_scan_reduced_size_everywhere(orc):
    # Mamba-130M-shaped recipe at a size the oracle covers in full:
    # several chunks, several channel groups and a ragged channel tail
    w = W.WORKLOADS["mamba130m_layer"]
    inp = _gen(w, batch=2, seqlen=600, dim=200)
    _say("case mamba130m recipe B=2 L=600 D=200 bf16, automatic plan")
    y, hL = _run(inp)
    _full_compare(orc, inp, y, hL, TOL["bf16"], "reduced layer scan")


def test_million_length_full_size_sampled(orc):
    w = W.WORKLOADS["million_length"]
    _say(f"case million_length B=1 L={w.seqlen} D={w.dim} N=16 bf16: generating inputs")
    inp = W.generate_scan(w, device=DEV)
    _say("case million_length: scanning (automatic plan)")
    y, hL = _run(inp)
    idx = sample_channels(w.dim, count=8, seed=w.seed)
    _say(f"case million_length: oracle on {len(idx)} channels")
    yo, ho = oracle_on_channels(orc, inp, idx)
    ix = torch.as_tensor(idx, device=DEV)
    assert_close(y.index_select(2, ix), yo, TOL["bf16"], "million_length y (sampled channels)")
    assert_close(hL.index_select(1, ix), ho, TOL["bf16"], "million_length hL (sampled channels)")
    del inp, y, hL
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", [0, 37])
def test_decode_layer_full_size(orc, layer):
    w = W.WORKLOADS["decode_64layer"]
    d = {k: v.to(DEV) for k, v in W.generate_decode_layer(w, layer).items()}
    h_before = d["h"].clone()
    _say(f"case decode layer {layer}: batch {w.batch} D {w.dim} N {w.dstate} bf16")
    y = ms.state_update(d["h"], d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"])
    torch.cuda.synchronize()
    yo, ho = orc.state_update(h_before, d["x"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"])
    assert_close(y, yo, TOL["bf16"], "decode y")
    assert_close(d["h"], ho, TOL["bf16"], "decode state")


# ---------------------------------------------------------------------------
# shapes, options and edge cases


CASES = [
    # (batch, seqlen, dim, dstate, io)
    (1, 1, 1, 1, "f32"),
    (2, 2, 3, 16, "f32"),
    (1, 7, 65, 16, "f32"),
    (2, 8, 64, 16, "bf16"),
    (3, 9, 130, 4, "f32"),
    (2, 63, 100, 8, "bf16"),
    (1, 65, 64, 3, "bf16"),
    (2, 257, 129, 16, "f32"),
    (1, 1000, 96, 16, "bf16"),
    (4, 300, 40, 5, "f32"),
    (1, 129, 300, 1, "f32"),
    (2, 77, 64, 2, "bf16"),
]


def _case_inputs(batch, seqlen, dim, dstate, io, seed, h0=True):
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = W.io_torch_dtype(io)

    def n(*s):
        return torch.randn(*s, generator=g)
    inp = dict(
        x=n(batch, seqlen, dim).to(dt),
        delta=torch.nn.functional.softplus(n(batch, seqlen, dim) - 1.0).to(dt),
        A=-torch.exp(torch.rand(dim, dstate, generator=g) * 2 - 1),
        B=n(batch, seqlen, dstate).to(dt), C=n(batch, seqlen, dstate).to(dt),
        D=n(dim), z=n(batch, seqlen, dim).to(dt),
        h0=n(batch, dim, dstate) if h0 else None)
    return {k: (v.to(DEV) if v is not None else None) for k, v in inp.items()}


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_shapes(orc, case):
    batch, seqlen, dim, dstate, io = case
    inp = _case_inputs(*case, seed=sum(case[:4]))
    _say(f"case shape {case}")
    y, hL = _run(inp)
    _full_compare(orc, inp, y, hL, TOL[io], f"shape {case}")


@pytest.mark.parametrize("chunk_len", [1, 5, 8, 16, 24, 100, 333, 1000])
def test_forced_chunk_lengths(orc, chunk_len):
    # every split of the sequence into parallel chunks gives the oracle's result
    inp = _case_inputs(2, 999, 72, 16, "f32", seed=5)
    _say(f"case chunk_len={chunk_len} B=2 L=999 D=72 N=16 fp32")
    y, hL = _run(inp, chunk_len=chunk_len)
    _full_compare(orc, inp, y, hL, TOL["f32"], f"chunk_len {chunk_len}")


SPLITS = [(16, s) for s in (1, 2, 4, 8)] + [(8, s) for s in (1, 2, 4, 8)] + \
         [(4, s) for s in (1, 2, 4)]


@pytest.mark.parametrize("dstate,split", SPLITS, ids=lambda v: str(v))
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_state_splits(orc, dstate, split, io):
    # every division of a channel's states over waves, with and without
    # sequence chunks, and a ragged last tile and channel group
    inp = _case_inputs(2, 203, 100, dstate, io, seed=dstate * 10 + split)
    yo, ho = orc.scan_fwd(**inp)
    for chunk_len in (0, 24, 203):
        _say(f"case N={dstate} split={split} chunk_len={chunk_len} {io}")
        y, hL = _run(inp, chunk_len=chunk_len, state_split=split)
        assert_close(y, yo, TOL[io], f"N={dstate} split={split} chunk={chunk_len} y")
        assert_close(hL, ho, TOL[io], f"N={dstate} split={split} chunk={chunk_len} hL")


def test_split_plan_choices_agree():
    # different plans of one large scan agree closely with each other
    w = W.WORKLOADS["mamba28b_layer"]
    inp = W.generate_scan(w, device=DEV, batch=2, seqlen=512, dim=1024)
    ref, href = _run(inp, chunk_len=512, state_split=1)
    for split in (2, 4, 8):
        for chunk_len in (64, 512):
            _say(f"case plan agreement split={split} chunk_len={chunk_len}")
            y, hL = _run(inp, chunk_len=chunk_len, state_split=split)
            assert_close(y, ref.float(), TOL["bf16"], f"split {split} chunk {chunk_len} vs 1/512")
            assert_close(hL, href, 1e-4, f"split {split} chunk {chunk_len} state")


def test_optional_inputs(orc):
    base = _case_inputs(2, 50, 70, 16, "f32", seed=9)
    for drop in (("z",), ("D",), ("h0",), ("z", "D", "h0")):
        inp = dict(base)
        for k in drop:
            inp[k] = None
        _say(f"case without {drop}")
        y, hL = _run(inp)
        _full_compare(orc, inp, y, hL, TOL["f32"], f"without {drop}")
    _say("case without hL")
    y, hL = _run(base, return_state=False)
    assert hL is None
    yo, _ = orc.scan_fwd(**base)
    assert_close(y, yo, TOL["f32"], "y without hL")


def test_state_aliasing_h0_and_hL(orc):
    for chunk_len in (0, 16):
        inp = _case_inputs(2, 200, 90, 16, "f32", seed=11)
        yo, ho = orc.scan_fwd(**inp)
        h = inp["h0"]
        _say(f"case hL aliases h0, chunk_len={chunk_len}")
        y, hL = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                            inp["z"], h, state_out=h, chunk_len=chunk_len)
        torch.cuda.synchronize()
        assert hL.data_ptr() == h.data_ptr()
        assert_close(y, yo, TOL["f32"], "aliased y")
        assert_close(h, ho, TOL["f32"], "aliased state")


def test_empty_sequence_copies_state():
    inp = _case_inputs(2, 0, 33, 16, "bf16", seed=1)
    _say("case seqlen 0")
    y, hL = _run(inp)
    assert y.shape == (2, 0, 33)
    assert torch.equal(hL, inp["h0"])
    inp["h0"] = None
    y, hL = _run(inp)
    assert torch.count_nonzero(hL) == 0


def test_empty_batch_and_dim():
    for b, d in ((0, 16), (2, 0)):
        inp = _case_inputs(b, 5, d, 4, "f32", seed=2)
        y, hL = _run(inp)
        assert y.numel() == 0 and hL.numel() == 0


def test_split_sequence_resumes_from_state(orc):
    # scanning [0, m) then [m, L) from the returned state equals one scan
    inp = _case_inputs(2, 700, 130, 16, "bf16", seed=3)
    y, hL = _run(inp)
    m = 333
    first = {k: (v[:, :m].contiguous() if k in ("x", "delta", "B", "C", "z") else v)
             for k, v in inp.items()}
    second = {k: (v[:, m:].contiguous() if k in ("x", "delta", "B", "C", "z") else v)
              for k, v in inp.items()}
    y1, h1 = _run(first)
    second["h0"] = h1
    y2, h2 = _run(second)
    yo, ho = orc.scan_fwd(**inp)
    assert_close(torch.cat([y1, y2], dim=1), yo, TOL["bf16"], "split y")
    assert_close(h2, ho, TOL["bf16"], "split state")


def test_decode_steps_equal_scan(orc):
    inp = _case_inputs(3, 12, 100, 16, "f32", seed=4)
    yo, ho = orc.scan_fwd(**inp)
    h = inp["h0"].clone()
    ys = []
    for t in range(12):
        ys.append(ms.state_update(h, inp["x"][:, t].contiguous(), inp["delta"][:, t].contiguous(),
                                  inp["A"], inp["B"][:, t].contiguous(),
                                  inp["C"][:, t].contiguous(), inp["D"],
                                  inp["z"][:, t].contiguous()))
    torch.cuda.synchronize()
    assert_close(torch.stack(ys, dim=1), yo, TOL["f32"], "decode steps y")
    assert_close(h, ho, TOL["f32"], "decode steps state")


@pytest.mark.parametrize("dstate", [1, 3, 4, 8, 12, 16])
def test_decode_shapes(orc, dstate):
    for io in ("f32", "bf16"):
        inp = _case_inputs(5, 1, 77, dstate, io, seed=dstate)
        h = inp["h0"].clone()
        y = ms.state_update(h, inp["x"][:, 0].contiguous(), inp["delta"][:, 0].contiguous(),
                            inp["A"], inp["B"][:, 0].contiguous(), inp["C"][:, 0].contiguous(),
                            inp["D"], inp["z"][:, 0].contiguous())
        torch.cuda.synchronize()
        yo, ho = orc.scan_fwd(**inp)
        assert_close(y, yo[:, 0], TOL[io], f"decode N={dstate} {io} y")
        assert_close(h, ho, TOL[io], f"decode N={dstate} {io} state")


def test_bitwise_determinism():
    inp = _case_inputs(2, 1500, 300, 16, "bf16", seed=6)
    y1, h1 = _run(inp)
    y2, h2 = _run(inp)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_nan_propagates():
    inp = _case_inputs(1, 40, 64, 16, "f32", seed=7)
    inp["x"][0, 10, 5] = float("nan")
    y, hL = _run(inp)
    assert torch.isnan(y[0, 10:, 5]).all()
    assert torch.isfinite(y[0, :10]).all() and torch.isfinite(y[0, :, 6]).all()
