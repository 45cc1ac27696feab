"""CPU: the parts of bench.py's JSON contract that need no GPU.

The benchmark measures one GPU; asked for more it refuses with a message
before touching a device. Its algorithmic byte count for the Mamba-2.8B
layer is the sum of the tensors the scan must move, added up here from the
shapes one by one. Its roofline names the kernel the plan launches: the
mixed whole/half-group kernel when the plan splits channel groups, the
whole-group kernel otherwise.
"""
import os
import subprocess
import sys

import bench
import ssm_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_headline_algorithmic_bytes():
    w = W.WORKLOADS["mamba28b_layer"]
    b, l, d, n = 8, 2048, 5120, 16
    io = b * l * d * 2          # one of x, delta, z, y in bf16
    bc = b * l * n * 2          # one of B, C in bf16
    want = 4 * io + 2 * bc + d * n * 4 + d * 4 + b * d * n * 4   # + A, D, hL (h0 is zero)
    assert want == 675_106_816
    assert bench.algorithmic_bytes(w) == want
    # the fused activation reads one fp32 bias per channel more
    assert bench.algorithmic_bytes(w, softplus=True) == want + d * 4


def test_roofline_names_the_planned_kernel():
    import selective_state_space_40_amd as ms
    whole = ms.Plan(2048, 4, ms.CARRY_RERUN, 0, 0)
    mixed = ms.Plan(2048, 4, ms.CARRY_RERUN, 128, 0)
    assert bench.dominant_kernel(whole) == "chunk_output_kernel"
    assert bench.dominant_kernel(mixed) == "chunk_mixed_kernel"


def test_backward_algorithmic_counts():
    # per element: two forward state updates of 4 operations per state, 9 per
    # state walking back (lam, Abar lam, lam Abar h, dA, the A term of
    # d delta, sum of lam B, the readout, the dB and dC terms) and 22 per
    # element; transcendentals: the two updates' exps and the gate's exp and
    # reciprocal
    w = W.WORKLOADS["mamba28b_layer"]
    elems = 8 * 2048 * 5120
    assert bench.backward_alu_ops(w) == (8 * 16 + 9 * 16 + 22) * elems
    assert bench.backward_alu_ops(w, softplus=True) == (8 * 16 + 9 * 16 + 22 + 16) * elems
    assert bench.backward_transcendentals(w) == 2 * 16 + 2
    assert bench.backward_transcendentals(w, softplus=True) == 2 * 16 + 2 + 4
    # bytes: x, delta, z, dy in and dx, ddelta, dz out (bf16), B and C in
    # (bf16) and dB, dC out (fp32), A, D in and dA, dD out, dh0 out
    b, l, d, n = 8, 2048, 5120, 16
    want = 7 * b * l * d * 2 + 2 * b * l * n * (2 + 4) + 2 * (d * n * 4 + d * 4) + b * d * n * 4
    assert bench.backward_bytes(w) == want
