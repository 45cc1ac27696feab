"""GPU: one short run of bench.py and the fields of its JSON line.

The benchmark prints one line for the Mamba-2.8B-shaped layer scan (B=8,
L=2048, D=5120, N=16, bf16 I/O): throughput in elements/s, the HBM roofline
of the kernel the plan launches (algorithmic bytes per step against 8 TB/s,
the 60% target, the HBM traffic recorded from counters for this kernel's
sources), the vector issue fraction beside it, and the fp64 oracle timed on
the host as a reported baseline.
"""
import json
import os
import subprocess
import sys

import pytest
import torch

import bench

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_default_bench_line():
    print("case bench.py default workload, 3 steps", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                          "--warmup", "1", "--spin-up", "0.1", "--cpu-seconds", "1"],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout[-3000:]
    d = json.loads(lines[0])

    assert d["metric"] == bench.METRIC and d["unit"] == "elements/s"
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    c = d["config"]
    assert c["workload"] == "mamba28b_layer"
    assert (c["batch"], c["seqlen"], c["dim"], c["dstate"], c["io_dtype"]) == \
        (8, 2048, 5120, 16, "bf16")
    elems = 8 * 2048 * 5120
    assert d["value"] == pytest.approx(elems / (d["ms_per_step"] / 1e3), rel=1e-9)

    r = d["roofline"]
    # the HBM roofline the target is stated against: algorithmic bytes per
    # step over 8 TB/s
    w = bench_workload()
    nbytes = bench.algorithmic_bytes(w)
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["algorithmic_bytes"] == nbytes
    hbm = nbytes / (d["ms_per_step"] / 1e3) / 8e12
    assert r["frac"] == pytest.approx(hbm, abs=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-3)
    assert r["target_frac"] == 0.60 and r["target_met"] == (r["frac"] >= 0.60)
    assert 0.0 < r["frac"] < 1.0
    # beside it the vector issue fraction, one slot per fp32 operation, and
    # the HBM fraction at full issue (transcendentals at one slot and at two)
    iss = r["issue"]
    slots = bench.algorithmic_alu_ops(w)
    assert iss["algorithmic_slots"] == slots == 89 * elems
    assert iss["frac"] == pytest.approx(slots / (d["ms_per_step"] / 1e3) / 39.3216e12, abs=1e-3)
    assert 0.0 < iss["frac"] < 1.0
    # the same with each transcendental (N + 2 per element) at two issue cycles
    assert iss["algorithmic_slots_trans_at_2"] == (89 + 18) * elems
    assert iss["frac_trans_at_2"] == pytest.approx(
        (89 + 18) * elems / (d["ms_per_step"] / 1e3) / 39.3216e12, abs=1e-3)
    assert iss["frac"] < iss["frac_trans_at_2"] < 1.0
    assert iss["hbm_frac_at_full_issue"] == pytest.approx(
        (nbytes / 8e12) / (slots / 39.3216e12), abs=1e-3)
    assert iss["hbm_frac_at_full_issue_trans_at_2"] == pytest.approx(
        (nbytes / 8e12) / ((89 + 18) * elems / 39.3216e12), abs=1e-3)
    assert r["kernel"] in ("chunk_mixed_kernel", "chunk_output_kernel")
    # traffic comes from the counters recorded for this kernel's sources, or
    # is null once those sources have changed
    rec = bench.recorded_traffic("mamba28b_layer", r["kernel"])
    assert r["traffic"] == (rec if rec is None else pytest.approx(rec))

    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "elements/s"
    assert cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]


def bench_workload():
    import ssm_workloads as W
    return W.WORKLOADS["mamba28b_layer"]
