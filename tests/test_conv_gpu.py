"""GPU parity of the short causal convolution and its decode step, called
through the C ABI, against the fp64 CPU oracle on the same seeded inputs.

Outputs: max abs error <= 1e-5 * max|oracle| (fp32 I/O) or 2e-2 * max|oracle|
(bf16 I/O), as for the scan. The handed-on state holds inputs, which the
I/O dtype represents exactly, so it must match the oracle bit for bit.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import selective_state_space_40_amd as ms
import ssm_workloads as W
from parity_util import TOL, assert_close, sample_channels

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


def _state_equal(got, want_f64, what):
    want = torch.as_tensor(want_f64).to(got.dtype)
    assert torch.equal(got.cpu(), want), f"{what}: handed-on state differs"


def _inputs(batch, seqlen, dim, width, io, seed, state=True, bias=True):
    w = dataclasses.replace(W.CONV_WORKLOADS["conv_mamba28b_layer"], width=width, io=io)
    inp = W.generate_conv(w, device=DEV, batch=batch, seqlen=seqlen, dim=dim, seed=seed,
                          state="normal" if state else "zero")
    if not bias:
        inp["bias"] = None
    return inp


CASES = [
    # (batch, seqlen, dim, width, io)
    (1, 1, 4, 4, "f32"), (2, 2, 8, 4, "bf16"), (1, 3, 64, 4, "f32"), (2, 5, 3, 4, "bf16"),
    (3, 16, 256, 4, "bf16"), (2, 17, 260, 4, "f32"), (1, 33, 65, 3, "f32"),
    (2, 100, 130, 2, "bf16"), (1, 47, 128, 1, "f32"), (2, 64, 96, 3, "bf16"),
    (4, 31, 1028, 4, "bf16"), (1, 200, 12, 2, "f32"),
    # whole numbers of 16-token chunks: the last chunk hands on the state
    (2, 32, 64, 4, "f32"), (1, 48, 4, 3, "bf16"), (3, 64, 6, 2, "bf16"), (2, 16, 20, 1, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_conv_shapes(orc, case):
    batch, seqlen, dim, width, io = case
    for state in (True, False):
        for bias in (True, False):
            for silu in (True, False):
                inp = _inputs(*case, seed=sum(case[:4]), state=state, bias=bias)
                _say(f"case conv {case} state={state} bias={bias} silu={silu}")
                y, st = ms.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"],
                                      silu=silu)
                torch.cuda.synchronize()
                yo, so = orc.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"],
                                        silu=silu)
                assert_close(y, yo, TOL[io], f"conv {case} y")
                _state_equal(st, so, f"conv {case}")


def test_conv_full_size_sampled(orc):
    w = W.CONV_WORKLOADS["conv_mamba28b_layer"]
    inp = W.generate_conv(w, device=DEV)
    _say(f"case {w.name} B={w.batch} L={w.seqlen} D={w.dim} W={w.width} bf16")
    y, st = ms.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"])
    torch.cuda.synchronize()
    idx = sample_channels(w.dim, seed=w.seed)
    ix = torch.as_tensor(idx, device=DEV)
    yo, so = orc.conv1d_fwd(inp["x"].index_select(2, ix), inp["weight"].index_select(0, ix),
                            inp["bias"].index_select(0, ix), None)
    assert_close(y.index_select(2, ix), yo, TOL["bf16"], "full-size conv y (sampled)")
    _state_equal(st.index_select(1, ix), so, "full-size conv")


def test_conv_state_aliasing_and_split(orc):
    for io in ("f32", "bf16"):
        inp = _inputs(2, 90, 132, 4, io, seed=3)
        yo, so = orc.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"])
        for m in (0, 1, 2, 3, 17, 58, 74, 89, 90):
            _say(f"case conv split at {m} {io}, state handed on in place")
            state = inp["state_in"].clone()
            y1, _ = ms.conv1d_fwd(inp["x"][:, :m].contiguous(), inp["weight"], inp["bias"],
                                  state, state_out=state)
            y2, _ = ms.conv1d_fwd(inp["x"][:, m:].contiguous(), inp["weight"], inp["bias"],
                                  state, state_out=state)
            torch.cuda.synchronize()
            assert_close(torch.cat([y1, y2], dim=1), yo, TOL[io], f"conv split {m} y")
            _state_equal(state, so, f"conv split {m}")


def test_conv_decode_steps_equal_forward(orc):
    # even channel counts take the 2-channels-per-thread decode kernel, odd
    # ones the single-channel kernel; every width of both
    for io in ("f32", "bf16"):
        for width, dim in ((4, 70), (3, 70), (2, 70), (1, 70), (4, 37), (3, 37), (2, 37), (1, 37)):
            inp = _inputs(3, 12, dim, width, io, seed=width + dim)
            yo, so = orc.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"])
            state = inp["state_in"].clone()
            _say(f"case conv decode W={width} D={dim} {io}")
            ys = [ms.conv1d_update(state, inp["x"][:, t].contiguous(), inp["weight"],
                                   inp["bias"]) for t in range(12)]
            torch.cuda.synchronize()
            assert_close(torch.stack(ys, dim=1), yo, TOL[io], f"conv decode W={width} D={dim} y")
            _state_equal(state, so, f"conv decode W={width} D={dim}")


def test_conv_decode_many_rows(orc):
    # 70,001 batch rows of a few channels: more rows than a grid dimension
    # of 65,535 holds, even and odd channel counts
    for io, dim in (("bf16", 6), ("f32", 5)):
        inp = _inputs(70001, 1, dim, 4, io, seed=dim)
        yo, so = orc.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"])
        state = inp["state_in"].clone()
        _say(f"case conv decode 70001 rows D={dim} {io}")
        y = ms.conv1d_update(state, inp["x"][:, 0].contiguous(), inp["weight"], inp["bias"])
        torch.cuda.synchronize()
        assert_close(y, yo[:, 0], TOL[io], f"conv decode 70001 rows D={dim} y")
        _state_equal(state, so, f"conv decode 70001 rows D={dim}")


@pytest.mark.parametrize("layer", [0, 41])
def test_conv_decode_layer_full_size(orc, layer):
    w = W.CONV_WORKLOADS["conv_decode_64layer"]
    d = W.generate_conv_decode_layer(w, layer, device=DEV)
    before = d["state"].clone()
    _say(f"case conv decode layer {layer}: batch {w.batch} D {w.dim} W {w.width} bf16")
    y = ms.conv1d_update(d["state"], d["x"], d["weight"], d["bias"])
    torch.cuda.synchronize()
    yo, so = orc.conv1d_update(before, d["x"], d["weight"], d["bias"])
    assert_close(y, yo, TOL["bf16"], "conv decode layer y")
    _state_equal(d["state"], so, "conv decode layer")


def test_conv_empty_sequence_hands_on_state():
    inp = _inputs(2, 0, 40, 4, "bf16", seed=8)
    y, st = ms.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"])
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 40) and torch.equal(st, inp["state_in"])
    y, st = ms.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st) == 0


def test_conv_deterministic_and_nan():
    inp = _inputs(2, 300, 256, 4, "bf16", seed=9)
    y1, s1 = ms.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"])
    y2, s2 = ms.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    x = inp["x"].clone()
    x[0, 50, 7] = float("nan")
    y, _ = ms.conv1d_fwd(x, inp["weight"], inp["bias"], inp["state_in"])
    torch.cuda.synchronize()
    assert torch.isnan(y[0, 50:54, 7]).all()
    assert torch.isfinite(y[0, 54:, 7]).all() and torch.isfinite(y[0, :50, 7]).all()
    assert torch.isfinite(y[0, :, 8]).all()
