"""Workload shapes and input recipes against the numbers the pages print
(tests/golden/mamba_pages_numbers.json, each entry with its citation)."""
import json
import os

import torch

import ssm_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mamba_pages_numbers.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_decode_state_matches_mamba28b_state_size():
    g = _golden()["state_size"]
    w = W.WORKLOADS["decode_64layer"]
    assert (w.layers, w.dim, w.dstate) == (g["layers"], g["channels"], g["ssm_numbers_per_channel"])
    numbers = w.layers * w.dim * (w.dstate + g["conv_inputs_per_channel"])
    assert numbers == g["total_numbers"]
    assert round(numbers * 2 / 1e6, 1) == g["megabytes_at_16_bit"]


def test_layer_shape_is_mamba28b():
    g = _golden()
    w = W.WORKLOADS["mamba28b_layer"]
    assert (w.dim, w.dstate) == (g["state_size"]["channels"], g["default_state_size"]["dstate"])


def test_s4d_real_a_runs_from_minus1_to_minus16():
    g = _golden()["a_init"]
    w = W.WORKLOADS["mamba28b_layer"]
    inp = W.generate_scan(w, batch=1, seqlen=2, dim=3)
    A = inp["A"]
    assert A.shape == (3, g["count"])
    assert torch.all(A[:, 0] == g["first"]) and torch.all(A[:, -1] == g["last"])
    assert torch.all(A[:, 1:] < A[:, :-1])


def test_recipe_distributions_and_determinism():
    w = W.WORKLOADS["mamba130m_layer"]
    a = W.generate_scan(w, batch=2, seqlen=256, dim=64)
    b = W.generate_scan(w, batch=2, seqlen=256, dim=64)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    assert a["x"].dtype == torch.bfloat16 and a["A"].dtype == torch.float32
    assert torch.all(a["delta"].float() > 0)
    assert torch.all(a["A"] < 0)
    assert abs(float(a["x"].float().std()) - 1.0) < 0.05
    assert a["h0"] is None
    tiny = W.generate_scan(W.WORKLOADS["tiny_f32"])
    assert tiny["x"].shape == (1, 64, 16) and tiny["A"].shape == (16, 4)
    assert tiny["x"].dtype == torch.float32


def test_decode_layers_are_distinct():
    w = W.WORKLOADS["decode_64layer"]
    l0 = W.generate_decode_layer(w, 0, batch=4, dim=32)
    l1 = W.generate_decode_layer(w, 1, batch=4, dim=32)
    assert l0["h"].shape == (4, 32, 16) and l0["B"].shape == (4, 16)
    assert not torch.equal(l0["x"], l1["x"])


def test_conv_workloads_keep_the_last_4_inputs_per_channel():
    g = _golden()["state_size"]
    for name in ("conv_mamba28b_layer", "conv_decode_64layer"):
        w = W.CONV_WORKLOADS[name]
        assert w.width == g["conv_inputs_per_channel"] and w.dim == g["channels"]
    assert W.CONV_WORKLOADS["conv_decode_64layer"].layers == g["layers"]
    a = W.generate_conv(W.CONV_WORKLOADS["conv_mamba28b_layer"], batch=1, seqlen=5, dim=8)
    b = W.generate_conv(W.CONV_WORKLOADS["conv_mamba28b_layer"], batch=1, seqlen=5, dim=8)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["weight"], b["weight"])
    assert a["state_in"] is None and a["x"].dtype == torch.bfloat16
    assert float(a["weight"].abs().max()) <= 0.5
