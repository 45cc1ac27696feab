"""GPU: the entry points inside captured HIP graphs.

Decode steps are replayed as graphs (bench.py does so for the 64-layer
decode workloads), so every entry point a decode step or a chunked scan
uses is captured here and replayed several times, with eager work and
synchronisations between the replays, and every replay is compared bit for
bit with the same calls made eagerly on copies of the same state (the same
kernels on the same inputs give the same bits). Nothing captured may record
a memset or allocate outside the capture's pool; a failure here means a
captured node does not do on replay what it did when captured.
"""
import dataclasses
import sys

import pytest
import torch

import selective_state_space_40_amd as ms
import ssm_workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 4


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


def _capture(fn):
    """Warm `fn` on a side stream, then capture it; returns the graph."""
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def _eager_noise(k):
    # unrelated eager work between replays: a reduction and a scan of its own
    a = torch.randn(1 << 16, device=DEV, generator=torch.Generator(DEV).manual_seed(k))
    (a * a).sum().item()
    inp = {kk: (v.to(DEV) if v is not None else None)
           for kk, v in W.generate_scan(W.WORKLOADS["tiny_f32"], seed=100 + k).items()}
    ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                inp["h0"])
    torch.cuda.synchronize()


def test_graph_decode_layers_replay_bitwise():
    """Three layers of ssm_state_update and causal_conv1d_update per step."""
    w = W.WORKLOADS["decode_64layer"]
    cw = W.CONV_WORKLOADS["conv_decode_64layer"]
    layers = [{k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
               for k, v in W.generate_decode_layer(w, l, batch=8, dim=320).items()}
              for l in range(3)]
    convs = [{k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
              for k, v in W.generate_conv_decode_layer(cw, l, batch=8, dim=320).items()}
             for l in range(3)]
    ys = [torch.empty_like(L["x"]) for L in layers]
    cys = [torch.empty_like(C["x"]) for C in convs]

    def step():
        for C, cy in zip(convs, cys):
            ms.conv1d_update(C["state"], C["x"], C["weight"], C["bias"], out=cy)
        for L, y in zip(layers, ys):
            ms.state_update(L["h"], L["x"], L["delta"], L["A"], L["B"], L["C"], L["D"], L["z"],
                            out=y)

    # eager twins of the states, advanced alongside the replays
    h_ref = [L["h"].clone() for L in layers]
    s_ref = [C["state"].clone() for C in convs]
    graph = _capture(step)
    torch.cuda.synchronize()
    # capture warmed up once and captured once: the states advanced once (the
    # captured call does not run); bring the twins to the same point
    for C, s in zip(convs, s_ref):
        ms.conv1d_update(s, C["x"], C["weight"], C["bias"])
    for L, h in zip(layers, h_ref):
        ms.state_update(h, L["x"], L["delta"], L["A"], L["B"], L["C"], L["D"], L["z"])
    torch.cuda.synchronize()
    for L, h in zip(layers, h_ref):
        assert torch.equal(L["h"], h)
    for r in range(REPLAYS):
        _say(f"case graph decode: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        for C, s, cy in zip(convs, s_ref, cys):
            y_ref = ms.conv1d_update(s, C["x"], C["weight"], C["bias"])
            assert torch.equal(cy, y_ref), f"conv y, replay {r}"
            assert torch.equal(C["state"], s), f"conv state, replay {r}"
        for L, h, y in zip(layers, h_ref, ys):
            y_ref = ms.state_update(h, L["x"], L["delta"], L["A"], L["B"], L["C"], L["D"], L["z"])
            assert torch.equal(y, y_ref), f"decode y, replay {r}"
            assert torch.equal(L["h"], h), f"decode state, replay {r}"
        _eager_noise(r)


def test_graph_chunked_scan_and_ssd_replay_bitwise():
    """A scan forced into several chunks, once with the summary-pass carry and
    once with the repaired carry (whose head reruns stop on the data), each
    with a workspace allocated while capturing, a single-chunk scan with
    whole and half channel groups, and a dual-form call."""
    w = W.WORKLOADS["mamba130m_layer"]
    inp = {k: (v.to(DEV) if v is not None else None)
           for k, v in W.generate_scan(w, batch=2, seqlen=300, dim=192, seed=11).items()}
    # delta ~ softplus(N(0,1)): the repaired carry's head reruns stop inside
    # the 104-token chunks
    fast = {k: (v.to(DEV) if v is not None else None)
            for k, v in W.generate_scan(dataclasses.replace(w, delta_shift=0.0), batch=2,
                                        seqlen=300, dim=192, seed=13).items()}
    sw = W.SSD_WORKLOADS["ssd_mamba2_layer"]
    sinp = {k: (v.to(DEV) if v is not None else None)
            for k, v in W.generate_ssd(sw, batch=2, seqlen=150, nheads=2, dstate=128,
                                       seed=12).items()}
    y = torch.empty_like(inp["x"])
    hL = torch.empty(2, 192, w.dstate, dtype=torch.float32, device=DEV)
    ry = torch.empty_like(inp["x"])
    rhL = torch.empty_like(hL)
    my = torch.empty_like(inp["x"])
    mhL = torch.empty_like(hL)
    sy = torch.empty_like(sinp["x"])
    shL = torch.empty(2, 2, 64, 128, dtype=torch.float32, device=DEV)

    def step():
        ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], chunk_len=64, out=y, state_out=hL)
        ms.scan_fwd(fast["x"], fast["delta"], fast["A"], fast["B"], fast["C"], fast["D"],
                    fast["z"], fast["h0"], chunk_len=104, carry=ms.CARRY_REPAIR, out=ry,
                    state_out=rhL)
        # one chunk, whole and half channel groups in one launch
        ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], chunk_len=300, state_split=4, halves=3, out=my, state_out=mhL)
        ms.ssd_fwd(sinp["x"], sinp["dt"], sinp["A"], sinp["B"], sinp["C"], sinp["D"], sinp["z"],
                   sinp["h0"], out=sy, state_out=shL)

    graph = _capture(step)
    y_ref, h_ref = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                               inp["z"], inp["h0"], chunk_len=64)
    ry_ref, rh_ref = ms.scan_fwd(fast["x"], fast["delta"], fast["A"], fast["B"], fast["C"],
                                 fast["D"], fast["z"], fast["h0"], chunk_len=104,
                                 carry=ms.CARRY_REPAIR)
    my_ref, mh_ref = ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                 inp["z"], inp["h0"], chunk_len=300, state_split=4, halves=3)
    sy_ref, sh_ref = ms.ssd_fwd(sinp["x"], sinp["dt"], sinp["A"], sinp["B"], sinp["C"],
                                sinp["D"], sinp["z"], sinp["h0"])
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        _say(f"case graph chunked scan + ssd: replay {r}")
        y.zero_()
        ry.zero_()
        my.zero_()
        sy.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hL, h_ref), f"chunked scan, replay {r}"
        assert torch.equal(ry, ry_ref) and torch.equal(rhL, rh_ref), f"repaired carry, replay {r}"
        assert torch.equal(my, my_ref) and torch.equal(mhL, mh_ref), f"half groups, replay {r}"
        assert torch.equal(sy, sy_ref) and torch.equal(shL, sh_ref), f"ssd, replay {r}"
        _eager_noise(r)


def test_graph_backward_replay_bitwise():
    """The backward pass captured twice: a sequence cut into chunks (state
    and adjoint summaries, their folds, the reverse kernel, the reductions;
    workspace allocated while capturing) and a whole sequence with half
    channel groups."""
    w = dataclasses.replace(W.WORKLOADS["mamba130m_layer"], h0="normal")
    inp = {k: (v.to(DEV) if v is not None else None)
           for k, v in W.generate_scan(w, batch=2, seqlen=300, dim=192, seed=21).items()}
    g = torch.Generator(device=DEV).manual_seed(22)
    dy = torch.randn(2, 300, 192, generator=g, device=DEV).to(inp["x"].dtype)
    dhL = torch.randn(2, 192, w.dstate, generator=g, device=DEV)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["h0"])
    out = {}

    def step():
        out["cut"] = ms.scan_bwd(*args, dy=dy, dhL=dhL, chunk_len=64)
        out["half"] = ms.scan_bwd(*args, dy=dy, dhL=dhL, chunk_len=304, halves=3)

    graph = _capture(step)
    ref = {"cut": ms.scan_bwd(*args, dy=dy, dhL=dhL, chunk_len=64),
           "half": ms.scan_bwd(*args, dy=dy, dhL=dhL, chunk_len=304, halves=3)}
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        _say(f"case graph backward: replay {r}")
        for grads in out.values():
            for v in grads.values():
                if v is not None:
                    v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for kind, grads in out.items():
            for k, v in grads.items():
                if v is None:
                    assert ref[kind][k] is None
                    continue
                assert torch.equal(v, ref[kind][k]), f"backward {kind} {k}, replay {r}"
        _eager_noise(r)
