"""Benchmark of the selective scan on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one ssm_scan_fwd over the whole workload (every kernel of the
fused scan: chunk summaries, carry combine, output pass), with inputs
already resident in HBM. The default workload is the Mamba-2.8B-shaped layer
scan (batch 8, 2,048 tokens, 5,120 channels, 16 states, bf16 I/O, fp32
state). Two input sets alternate between steps so no step reads inputs the
previous step left in the 256 MB last-level cache.

Prints one JSON line: scan elements/s (B*L*D) as `value`, the algorithmic
HBM bytes per second, the roofline of the dominant kernel (timed with HIP
events on the stream it runs on) and the fp64 CPU oracle timed on the host
cores over a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scan elements/s (B·L·D) and achieved HBM GB/s, Mamba-2.8B layer shape"
HBM_PEAK_GBPS = 8000.0
# fp32 vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one lane-op per
# lane per cycle (FMA, multiply, add, convert and transcendental issue alike)
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mamba28b_layer")
    p.add_argument("--chunk-len", type=int, default=0, help="0 = the library's automatic plan")
    p.add_argument("--state-split", type=int, default=0, help="0 = the library's automatic plan")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-channels", type=int, default=0,
                   help="channels of the CPU-baseline sample (0 = sized to ~10 s)")
    return p.parse_args()


def algorithmic_bytes(w):
    """Bytes the scan must move: x, delta, z in and y out (I/O dtype), B and C
    in, A and D in (fp32), final state out (fp32), initial state in when the
    workload has one. The expanded (B, L, D, N) state is never stored."""
    s = 4 if w.io == "f32" else 2
    b, l, d, n = w.batch, w.seqlen, w.dim, w.dstate
    total = 4 * b * l * d * s + 2 * b * l * n * s + d * n * 4 + d * 4 + b * d * n * 4
    if w.h0 == "normal":
        total += b * d * n * 4
    return total


def algorithmic_alu_ops(w):
    """fp32 lane-operations the scan must issue per element: per state one
    multiply for delta*A, one exponential, one multiply for (delta*x)*B, one
    FMA for the state update and one FMA for the readout; per element one
    multiply for delta*x, one FMA for the skip term, the gate (one multiply,
    one exponential, one add, one reciprocal, two multiplies) and one
    conversion to the I/O dtype."""
    n = w.dstate
    per_elem = 5 * n + 1 + 1 + 6 + (1 if w.io == "bf16" else 0)
    return per_elem * w.batch * w.seqlen * w.dim


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import selective_state_space_40_amd as ms
    import ssm_workloads as W

    w = W.WORKLOADS[args.workload]
    assert w.kind == "scan", "bench.py times scan workloads"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.load_library()

    sets = [W.generate_scan(w, device=dev, seed=w.seed + 101 * i) for i in range(2)]
    y = torch.empty_like(sets[0]["x"])
    hL = torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev)

    def step(i):
        inp = sets[i % 2]
        ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], chunk_len=args.chunk_len, state_split=args.state_split, out=y,
                    state_out=hL)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # the plan the library chose, for the record
    chunk_len, split, _ = ms.resolve_plan(w.batch, w.seqlen, w.dim, w.dstate,
                                          W.io_torch_dtype(w.io), args.chunk_len,
                                          args.state_split)
    nchunks = -(-w.seqlen // chunk_len)

    elems = w.batch * w.seqlen * w.dim
    sec = ms_per_step / 1e3
    value = elems / sec
    bytes_alg = algorithmic_bytes(w)
    gbps = bytes_alg / sec / 1e9
    ops = algorithmic_alu_ops(w)
    tops = ops / sec / 1e12

    # Dominant kernel: the output pass. With a single chunk the step is that
    # one kernel; otherwise the step also holds the summary and carry passes
    # and the figure below is the whole step, a lower bound for the kernel.
    hbm_frac = gbps / HBM_PEAK_GBPS
    alu_frac = tops / ALU_PEAK_TOPS
    bound = "alu" if ops / (ALU_PEAK_TOPS * 1e12) > bytes_alg / (HBM_PEAK_GBPS * 1e9) else "hbm"
    roofline = {
        "bound": bound,
        "achieved": round(tops if bound == "alu" else gbps, 3),
        "peak": ALU_PEAK_TOPS if bound == "alu" else HBM_PEAK_GBPS,
        "unit": "Tops/s (fp32 lane-ops)" if bound == "alu" else "GB/s",
        "frac": round(alu_frac if bound == "alu" else hbm_frac, 4),
        "traffic": None,
        "kernel": "chunk_output_kernel" if nchunks == 1 else "ssm_scan_fwd step (all passes)",
        "hbm_GBps": round(gbps, 1),
        "hbm_frac": round(hbm_frac, 4),
    }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, sets[0], args.cpu_sample_channels)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "io_dtype": w.io, "chunk_len": int(chunk_len),
                   "nchunks": int(nchunks), "state_split": int(split),
                   "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1),
        "wall_s": round(wall, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, inp, channels):
    """The fp64 oracle, as it is, on the host over a channel sample of the
    same workload (all batch rows, all tokens)."""
    import numpy as np
    import torch

    import oracle

    orc = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    if channels <= 0:
        # about 10 s at ~1e7 elements/s per core
        per_core = 1.0e7
        channels = int(10.0 * per_core * threads / (w.batch * w.seqlen))
        channels = max(8, min(w.dim, channels))
    idx = torch.arange(channels, device=inp["x"].device)
    sub = {k: v for k, v in dict(
        x=inp["x"].index_select(2, idx), delta=inp["delta"].index_select(2, idx),
        A=inp["A"].index_select(0, idx), B=inp["B"], C=inp["C"], D=inp["D"].index_select(0, idx),
        z=inp["z"].index_select(2, idx), h0=None).items()}
    host = {k: (oracle._f64(v) if v is not None else None) for k, v in sub.items()}
    t0 = time.perf_counter()
    orc.scan_fwd(**host)
    dt = time.perf_counter() - t0
    elems = w.batch * w.seqlen * channels
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: all {w.batch} batch rows x {w.seqlen} tokens x first "
                      f"{channels} of {w.dim} channels, fp64, {dt:.2f} s"}


if __name__ == "__main__":
    main()
