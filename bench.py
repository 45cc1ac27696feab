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
# The scan's target: 60% of peak HBM bandwidth on the Mamba-2.8B layer.
HBM_TARGET_FRAC = 0.60
# Vector issue budget: 256 CUs x 4 SIMDs, each issuing one wave64 vector
# instruction per quad-cycle (16 lanes x 4 cycles), at 2.4 GHz: 64 lane-slots
# per CU per clock. The kernels are built without packed fp32 forms, so an
# fp32 FMA, multiply, add or conversion takes one lane-slot. A
# transcendental (exp, log, reciprocal) keeps the transcendental unit busy
# for two quad-cycles, but other vector instructions can issue in the second
# (rocprofv3 counts that quad-cycle as SQ_ACTIVE_INST_VALU2): measured at
# 8 waves per SIMD, one exp among four independent FMAs cost 1.15 FMA
# issues, exps back to back 1.8. So a transcendental costs between one and
# two lane-slots; the issue roofline takes one (the instruction count) and
# reports the HBM fraction at full issue for both prices.
ISSUE_PEAK_T = 256 * 4 * 16 * 2.4e9 / 1e12
ALU_PEAK_TOPS = ISSUE_PEAK_T


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mamba28b_layer")
    p.add_argument("--chunk-len", type=int, default=0, help="0 = the library's automatic plan")
    p.add_argument("--state-split", type=int, default=0, help="0 = the library's automatic plan")
    p.add_argument("--carry", choices=("auto", "rerun", "repair"), default="auto",
                   help="how chunks of a cut sequence join (auto = the library's plan)")
    p.add_argument("--halves", type=int, default=0,
                   help="channel groups run as two 32-channel halves (0 = the library's plan, "
                        "-1 = none, k = the last k groups)")
    p.add_argument("--batch", type=int, default=0, help="override the workload's batch (0 = keep)")
    p.add_argument("--dim", type=int, default=0, help="override the workload's channels (0 = keep)")
    p.add_argument("--backward", action="store_true",
                   help="time ssm_scan_bwd (gradients of every input, states recomputed) "
                        "instead of the forward scan")
    p.add_argument("--delta-softplus", action="store_true",
                   help="pass delta before its activation with a per-channel bias and let the "
                        "kernels apply bias and softplus")
    p.add_argument("--spin-up", type=float, default=0.3,
                   help="seconds the step runs untimed before the warm-up steps, so the GPU "
                        "clock has left idle (0 = none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-channels", type=int, default=0,
                   help="channels of the CPU-baseline sample (0 = sized to ~10 s)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="the CPU baseline repeats its sample until this much wall time has "
                        "gone by (a sample that takes longer runs once)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy, for counter calibration")
    p.add_argument("--record-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                         "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE counter CSVs of the scan and of "
                        "the calibration copy into profiles/traffic_<workload>.json")
    return p.parse_args()


def algorithmic_bytes(w, softplus=False):
    """Bytes the scan must move: x, delta, z in and y out (I/O dtype), B and C
    in, A and D in (fp32), final state out (fp32), initial state in when the
    workload has one, the delta bias (fp32) with the fused activation. The
    expanded (B, L, D, N) state is never stored."""
    s = 4 if w.io == "f32" else 2
    b, l, d, n = w.batch, w.seqlen, w.dim, w.dstate
    total = 4 * b * l * d * s + 2 * b * l * n * s + d * n * 4 + d * 4 + b * d * n * 4
    if w.h0 == "normal":
        total += b * d * n * 4
    if softplus:
        total += d * 4
    return total


def transcendentals(w, softplus=False):
    """Transcendental lane-operations per element among algorithmic_alu_ops:
    the N exponentials, the gate's exponential and reciprocal, and with the
    fused activation softplus's exponential, logarithm and reciprocal."""
    return w.dstate + 2 + (3 if softplus else 0)


def issue_roofline(slots, sec):
    """Issue-slot fraction: algorithmic lane-slots (one per operation, a
    transcendental included) issued per second against ISSUE_PEAK_T."""
    achieved = slots / sec / 1e12
    return {"achieved": round(achieved, 3), "peak": ISSUE_PEAK_T,
            "unit": "T lane-issue-slots/s (one per fp32 operation)",
            "frac": round(achieved / ISSUE_PEAK_T, 4), "algorithmic_slots": slots}


def algorithmic_alu_ops(w, softplus=False):
    """fp32 lane-operations the scan must issue per element: per state one
    multiply for delta*A, one exponential, one multiply for (delta*x)*B, one
    FMA for the state update and one FMA for the readout; per element one
    multiply for delta*x, one FMA for the skip term, the gate (one multiply,
    one exponential, one add, one reciprocal, two multiplies) and one
    conversion to the I/O dtype. The fused activation adds per element the
    bias add and softplus: |v| scaling, exponential, add, compare, logarithm,
    three multiplies, reciprocal, subtract, max and add (12)."""
    n = w.dstate
    per_elem = 5 * n + 1 + 1 + 6 + (1 if w.io == "bf16" else 0) + (13 if softplus else 0)
    return per_elem * w.batch * w.seqlen * w.dim


COPY_BYTES = 1 << 30
# The kernel of a single-chunk scan: one launch of whole channel groups, or
# of whole and half groups when the plan splits some.
KERNEL_WHOLE = "chunk_output_kernel"
KERNEL_MIXED = "chunk_mixed_kernel"


def dominant_kernel(plan):
    return KERNEL_MIXED if plan.halves > 0 else KERNEL_WHOLE
KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_40_amd", "csrc", f)
                  for f in ("internal.h", "device_common.h", "scan_chunked.h", "scan_variant.hip")]


def source_hash():
    """Digest of the sources the scan kernels are compiled from: recorded
    counters are only used for the kernel they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def _counter_per_dispatch(csv_path, name, kernel_substr):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == name and kernel_substr in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no {name} rows for kernels matching {kernel_substr!r} in {csv_path}")
    vals.sort()
    return vals[len(vals) // 2]


def record_traffic(args):
    """HBM bytes per launch of the dominant kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a plain copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES)."""
    import csv
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.record_traffic
    names = {r["Kernel_Name"] for r in csv.DictReader(open(fetch_csv))}
    kernel = KERNEL_MIXED if any(KERNEL_MIXED in n for n in names) else KERNEL_WHOLE
    fetch = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel)
    write = _counter_per_dispatch(write_csv, "WRITE_SIZE", kernel)
    cfetch = _counter_per_dispatch(cfetch_csv, "FETCH_SIZE", "copy")
    cwrite = _counter_per_dispatch(cwrite_csv, "WRITE_SIZE", "copy")
    fetch_scale = COPY_BYTES / cfetch
    write_scale = COPY_BYTES / cwrite
    out = {"workload": args.workload, "kernel": kernel, "source_sha256_16": source_hash(),
           "fetch_bytes": fetch * fetch_scale, "write_bytes": write * write_scale,
           "traffic_bytes": fetch * fetch_scale + write * write_scale,
           "fetch_kib_raw": fetch, "write_kib_raw": write,
           "copy_fetch_kib_raw": cfetch, "copy_write_kib_raw": cwrite,
           "fetch_scale": fetch_scale, "write_scale": write_scale}
    with open(traffic_path(args.workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def calibrate_copy():
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": COPY_BYTES, "launches": 3}))


def recorded_traffic(workload, kernel):
    """Measured HBM bytes per launch, or None when not recorded, recorded
    for another kernel or recorded for a different kernel source."""
    try:
        with open(traffic_path(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_hash() or rec.get("kernel") != kernel:
        return None
    return rec.get("traffic_bytes")


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import selective_state_space_40_amd as ms
    import ssm_workloads as W

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload in W.SSD_WORKLOADS:
        bench_ssd(args, W.SSD_WORKLOADS[args.workload])
        return
    if args.workload in W.CONV_WORKLOADS:
        cw = W.CONV_WORKLOADS[args.workload]
        (bench_conv if cw.kind == "conv" else bench_conv_decode)(args, cw)
        return
    w = W.WORKLOADS[args.workload]
    if w.kind == "decode":
        bench_decode(args, w)
        return
    if args.backward:
        bench_backward(args, w)
        return
    if args.batch or args.dim:
        import dataclasses
        w = dataclasses.replace(w, batch=args.batch or w.batch, dim=args.dim or w.dim,
                                name=f"{w.name} resized")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.load_library()

    sp = args.delta_softplus
    sets = [W.generate_scan(w, device=dev, seed=w.seed + 101 * i, raw_delta=sp) for i in range(2)]
    y = torch.empty_like(sets[0]["x"])
    hL = torch.empty(w.batch, w.dim, w.dstate, dtype=torch.float32, device=dev)
    carry = {"auto": ms.CARRY_AUTO, "rerun": ms.CARRY_RERUN, "repair": ms.CARRY_REPAIR}[args.carry]

    def step(i):
        inp = sets[i % 2]
        ms.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], delta_bias=inp.get("delta_bias"), delta_softplus=sp,
                    chunk_len=args.chunk_len, state_split=args.state_split, carry=carry,
                    halves=args.halves, out=y, state_out=hL)

    _spin_up(step, args.spin_up)
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
    plan = ms.resolve_plan(w.batch, w.seqlen, w.dim, w.dstate, W.io_torch_dtype(w.io),
                           args.chunk_len, args.state_split, carry, args.halves)
    chunk_len, split = plan.chunk_len, plan.state_split
    nchunks = -(-w.seqlen // chunk_len)

    elems = w.batch * w.seqlen * w.dim
    sec = ms_per_step / 1e3
    value = elems / sec
    bytes_alg = algorithmic_bytes(w, sp)
    gbps = bytes_alg / sec / 1e9
    ops = algorithmic_alu_ops(w, sp)

    # Dominant kernel: the output pass (chunk_output_kernel, or
    # chunk_mixed_kernel when the plan splits channel groups). With a single
    # chunk the step is exactly that one launch, so the event time per step
    # is its launch duration; with several chunks the step also holds the
    # pass of chunk summaries (and the carry pass past 16 chunks) or the head
    # reruns, and the figure covers the whole step. Recorded traffic is used
    # only for the workload's own automatic plan.
    #
    # The roofline is HBM's, the one the target is stated against: the
    # fraction of 8 TB/s that the algorithmic bytes per step reach. Beside
    # it, the vector issue fraction and the HBM fraction this formulation
    # would reach with every issue slot busy (the step needs at least
    # algorithmic_slots / ISSUE_PEAK_T of issue time), with transcendentals
    # at one slot and, as a bound from the other side, at two; and the issue
    # fraction with every transcendental priced at the two issue cycles it
    # holds the vector ALU for (frac_trans_at_2).
    hbm_frac = gbps / HBM_PEAK_GBPS
    slots = ops
    issue = issue_roofline(slots, sec)
    slots2 = slots + transcendentals(w, sp) * elems
    issue["frac_trans_at_2"] = round(slots2 / sec / 1e12 / ISSUE_PEAK_T, 4)
    issue["algorithmic_slots_trans_at_2"] = slots2
    hbm_time = bytes_alg / (HBM_PEAK_GBPS * 1e9)
    issue["hbm_frac_at_full_issue"] = round(hbm_time / (slots / (ISSUE_PEAK_T * 1e12)), 4)
    issue["hbm_frac_at_full_issue_trans_at_2"] = round(
        hbm_time / (slots2 / (ISSUE_PEAK_T * 1e12)), 4)
    plain = not (args.batch or args.dim or sp or args.chunk_len or args.state_split or args.halves
                 or args.carry != "auto")
    traffic = recorded_traffic(w.name, dominant_kernel(plan)) if nchunks == 1 and plain else None
    roofline = {
        "bound": "hbm",
        "achieved": round(gbps, 3),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(hbm_frac, 4),
        "traffic": traffic,
        "kernel": dominant_kernel(plan) if nchunks == 1 else "ssm_scan_fwd step (all passes)",
        "algorithmic_bytes": bytes_alg,
        "target_frac": HBM_TARGET_FRAC,
        "target_met": hbm_frac >= HBM_TARGET_FRAC,
        "issue": issue,
        "algorithmic_ops": ops,
    }

    clock = gpu_clock_sample(step)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, sets[0], args.cpu_sample_channels, sp, args.cpu_seconds)

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
                   "carry": (None if nchunks == 1 else
                             {ms.CARRY_RERUN: "rerun", ms.CARRY_REPAIR: "repair"}[plan.carry]),
                   "half_groups": int(plan.halves),
                   "delta_activation": "bias + softplus in the kernels" if sp else
                                       "none (delta passed activated)",
                   "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1),
        "wall_s": round(wall, 4),
        "roofline": roofline,
        "gpu_clock": clock,
        "spin_up": dict(SPIN_UP),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def decode_bytes(w):
    """Bytes one decode step must move per layer: the fp32 state read and
    written, x, delta, z in and y out, B and C in, A and D in."""
    s = 4 if w.io == "f32" else 2
    b, d, n = w.batch, w.dim, w.dstate
    return 2 * b * d * n * 4 + 4 * b * d * s + 2 * b * n * s + d * n * 4 + d * 4


def bench_decode(args, w):
    """One step = one ssm_state_update per layer over all layers (each layer
    with its own state and inputs), replayed as a HIP graph so the launch
    rate of the host does not bound the timing."""
    import torch

    import selective_state_space_40_amd as ms
    import ssm_workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.load_library()
    layers = [{k: v.to(dev) for k, v in W.generate_decode_layer(w, l).items()}
              for l in range(w.layers)]
    ys = [torch.empty_like(L["x"]) for L in layers]

    def step():
        for L, y in zip(layers, ys):
            ms.state_update(L["h"], L["x"], L["delta"], L["A"], L["B"], L["C"], L["D"], L["z"],
                            out=y)

    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        step()  # warm the library and the allocator outside the capture
    torch.cuda.current_stream(dev).wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    _spin_up(lambda i: graph.replay(), args.spin_up)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream(dev)
    t0 = time.perf_counter()
    ev0.record(cur)
    for _ in range(args.steps):
        graph.replay()
    ev1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    sec = ms_per_step / 1e3
    elems = w.batch * w.dim * w.layers
    bytes_step = decode_bytes(w) * w.layers
    gbps = bytes_step / sec / 1e9
    clock = gpu_clock_sample(lambda i: graph.replay())
    line = {
        "metric": "decode state-update elements/s (batch*D*layers per step) and achieved HBM GB/s",
        "value": elems / sec, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                   "layers": w.layers, "io_dtype": w.io, "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1), "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "state_update_kernel (64 launches per step, graph replay)",
                     "algorithmic_bytes": bytes_step},
        "gpu_clock": clock,
        "spin_up": dict(SPIN_UP),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def backward_bytes(w, softplus=False):
    """Bytes the backward pass must move: x, delta, z, dy in and dx, ddelta,
    dz out (I/O dtype); B, C in (I/O dtype) and dB, dC out (fp32); A, D in,
    dA, dD out and dh0 out (fp32); the initial state in when there is one;
    with the fused activation the bias in and its gradient out."""
    s = 4 if w.io == "f32" else 2
    b, l, d, n = w.batch, w.seqlen, w.dim, w.dstate
    total = 7 * b * l * d * s + 2 * b * l * n * (s + 4) + 2 * (d * n * 4 + d * 4) + b * d * n * 4
    if w.h0 == "normal":
        total += b * d * n * 4
    if softplus:
        total += 2 * d * 4
    return total


def backward_alu_ops(w, softplus=False):
    """fp32 lane-operations the backward pass by recomputation must issue per
    element: the forward state update twice (once for the checkpoints, once
    to have every state while walking back: delta*A, exp, (delta*x)*B, FMA;
    4 per state each), and per state 9 in the walk back: the adjoint (FMA),
    its decayed hand-back Abar*lam (multiply), lam*Abar*h_prev (multiply),
    dA (FMA), the A term of d delta (FMA), sum of lam*B (FMA), the readout
    for dz (FMA), the dB and dC terms (a multiply each); per element about
    22 more (delta*x, dx and d delta from the sum of lam*B, the gate and its
    derivative, dx and readout skip terms, dD, conversions). The fused
    activation adds softplus and its derivative (16)."""
    n = w.dstate
    per_elem = 8 * n + 9 * n + 22 + (16 if softplus else 0)
    return per_elem * w.batch * w.seqlen * w.dim


def backward_transcendentals(w, softplus=False):
    """Transcendental lane-operations per element among backward_alu_ops: the
    exponential of each state update (twice; the walk back reuses the
    recomputation's decay factors), and the gate's exponential and
    reciprocal (sigmoid and silu share them); with the fused activation
    softplus's exponential, logarithm and reciprocal and its derivative's."""
    return 2 * w.dstate + 2 + (4 if softplus else 0)


def bench_backward(args, w):
    """One step = one ssm_scan_bwd over the whole workload: the checkpoint
    passes, the reverse kernel and the reductions, all in the timed region."""
    import torch

    import selective_state_space_40_amd as ms
    import ssm_workloads as W

    if args.batch or args.dim:
        import dataclasses
        w = dataclasses.replace(w, batch=args.batch or w.batch, dim=args.dim or w.dim,
                                name=f"{w.name} resized")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.load_library()
    sp = args.delta_softplus
    sets = []
    for i in range(2):
        inp = W.generate_scan(w, device=dev, seed=w.seed + 101 * i, raw_delta=sp)
        g = torch.Generator(device=dev).manual_seed(w.seed + 7 + i)
        inp["dy"] = torch.randn(w.batch, w.seqlen, w.dim, generator=g, device=dev).to(
            inp["x"].dtype)
        sets.append(inp)

    def step(i):
        inp = sets[i % 2]
        ms.scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                    inp["h0"], dy=inp["dy"], delta_bias=inp.get("delta_bias"),
                    delta_softplus=sp, halves=args.halves, chunk_len=args.chunk_len)

    ms_per_step, wall = _time_steps(step, args.warmup, args.steps, torch.cuda.current_stream(dev),
                                      args.spin_up)
    sec = ms_per_step / 1e3
    elems = w.batch * w.seqlen * w.dim
    nbytes = backward_bytes(w, sp)
    ops = backward_alu_ops(w, sp)
    slots = ops
    gbps = nbytes / sec / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline_backward(w, sets[0], sp, args.cpu_seconds)
    clock = gpu_clock_sample(step)
    plan = ms.resolve_bwd_plan(w.batch, w.seqlen, w.dim, w.dstate, W.io_torch_dtype(w.io),
                               args.chunk_len, args.halves)
    line = {
        "metric": "backward scan elements/s (B*L*D, all input gradients, states recomputed)",
        "value": elems / sec, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "dstate": w.dstate, "io_dtype": w.io, "checkpoint_every": 8,
                   "chunk_len": int(plan.chunk_len),
                   "nchunks": int(-(-w.seqlen // plan.chunk_len)),
                   "half_groups": int(plan.halves),
                   "delta_activation": "bias + softplus in the kernels" if sp else
                                       "none (delta passed activated)",
                   "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1), "wall_s": round(wall, 4),
        "roofline": dict(bound="alu", **issue_roofline(slots, sec),
                         traffic=None, kernel="ssm_scan_bwd step (all passes)",
                         algorithmic_bytes=nbytes, algorithmic_ops=ops,
                         hbm_GBps=round(gbps, 1), hbm_frac=round(gbps / HBM_PEAK_GBPS, 4)),
        "gpu_clock": clock,
        "spin_up": dict(SPIN_UP),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _oracle_passes(run, seconds):
    """Run one oracle pass over the sample, then more until `seconds` of wall
    time have gone by; returns (passes, seconds taken)."""
    passes, t0 = 0, time.perf_counter()
    while True:
        run()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return passes, dt


def _passes_text(passes, dt):
    return f"{passes} pass{'es' if passes > 1 else ''} in {dt:.1f} s"


def cpu_baseline_backward(w, inp, softplus, seconds):
    """The fp64 oracle's backward pass on the host over a channel sample (the
    per-channel work is independent; dB and dC come out as partial sums)."""
    import torch

    import oracle

    orc = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    # one pass sized to at most ~`seconds` at ~2e6 elements/s per core
    per_pass = max(seconds, 1.0) * 2.0e6 * threads
    channels = max(8, min(w.dim, int(per_pass / (w.batch * w.seqlen))))
    idx = torch.arange(channels, device=inp["x"].device)
    sub = dict(x=inp["x"].index_select(2, idx), delta=inp["delta"].index_select(2, idx),
               A=inp["A"].index_select(0, idx), B=inp["B"], C=inp["C"],
               D=inp["D"].index_select(0, idx), z=inp["z"].index_select(2, idx), h0=None,
               dy=inp["dy"].index_select(2, idx),
               delta_bias=inp["delta_bias"].index_select(0, idx) if softplus else None)
    host = {k: (oracle._f64(v) if v is not None else None) for k, v in sub.items()}
    passes, dt = _oracle_passes(lambda: orc.scan_bwd(**host, delta_softplus=softplus), seconds)
    elems = w.batch * w.seqlen * channels * passes
    return {"value": elems / dt, "unit": "elements/s",
            "cores": min(threads, w.batch), "kind": "oracle",
            "sample": f"{w.name}: all {w.batch} batch rows x {w.seqlen} tokens x first "
                      f"{channels} of {w.dim} channels, fp64 (rows in parallel), "
                      f"{_passes_text(passes, dt)}"}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores, MI355X


def ssd_flops(w):
    """Matrix-core flops the chunked dual form needs per chunk of Q = 64
    tokens and head of P = 64 channels (2 flops per multiply-add): C B^T on
    and below the diagonal (Q*Q*N/2), the masked matrix times x (Q*Q*P/2),
    C times the carried state (Q*N*P) and the state update (P*Q*N)."""
    q, p, n = 64, w.headdim, w.dstate
    per_chunk_head = q * q * n / 2 + q * q * p / 2 + q * n * p + p * q * n
    chunks = -(-w.seqlen // q)
    return 2.0 * per_chunk_head * chunks * w.batch * w.nheads


def ssd_bytes(w):
    """x, z in and y out, dt in (bf16), B and C in (bf16), A and D in, the
    final state out (fp32), the initial state in when there is one."""
    b, l, d, h, n = w.batch, w.seqlen, w.dim, w.nheads, w.dstate
    total = 3 * b * l * d * 2 + b * l * h * 2 + 2 * b * l * n * 2 + h * 4 + d * 4
    total += b * h * w.headdim * n * 4 * (2 if w.h0 == "normal" else 1)
    return total


def bench_ssd(args, w):
    """One step = one ssd_fwd over the whole workload (one launch)."""
    import torch

    import selective_state_space_40_amd as ms
    import ssm_workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.load_library()
    sets = [W.generate_ssd(w, device=dev, seed=w.seed + 101 * i) for i in range(2)]
    y = torch.empty_like(sets[0]["x"])
    hL = torch.empty(w.batch, w.nheads, w.headdim, w.dstate, dtype=torch.float32, device=dev)

    def step(i):
        inp = sets[i % 2]
        ms.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                   inp["h0"], out=y, state_out=hL)

    ms_per_step, wall = _time_steps(step, args.warmup, args.steps, torch.cuda.current_stream(dev),
                                      args.spin_up)
    sec = ms_per_step / 1e3
    flops = ssd_flops(w)
    nbytes = ssd_bytes(w)
    tflops = flops / sec / 1e12
    gbps = nbytes / sec / 1e9
    mfma_frac = tflops / MFMA_BF16_PEAK_TFLOPS
    hbm_frac = gbps / HBM_PEAK_GBPS
    bound = "mfma" if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBPS * 1e9) \
        else "hbm"
    cpu = None if args.no_cpu_baseline else cpu_baseline_ssd(w, sets[0], args.cpu_seconds)
    clock = gpu_clock_sample(step)
    line = {
        "metric": "Mamba-2 dual-form scan elements/s (B*L*D) and achieved HBM GB/s",
        "value": w.elements / sec, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "chunk": 64, "io_dtype": w.io,
                   "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1), "wall_s": round(wall, 4),
        "roofline": {"bound": bound,
                     "achieved": round(gbps if bound == "hbm" else tflops, 3),
                     "peak": HBM_PEAK_GBPS if bound == "hbm" else MFMA_BF16_PEAK_TFLOPS,
                     "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                     "frac": round(hbm_frac if bound == "hbm" else mfma_frac, 4),
                     "traffic": None, "kernel": "ssd_fwd_kernel",
                     "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                     "mfma_TFLOPs": round(tflops, 2), "mfma_frac": round(mfma_frac, 4),
                     "hbm_frac": round(hbm_frac, 4)},
        "gpu_clock": clock,
        "spin_up": dict(SPIN_UP),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_ssd(w, inp, seconds):
    """The fp64 oracle on the host over a sample of heads (heads are
    independent), all rows and tokens."""
    import torch

    import oracle

    orc = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    # one pass sized to at most ~`seconds` at ~4e6 elements/s per core
    per_pass = max(seconds, 1.0) * 4.0e6 * threads
    nh = max(1, min(w.nheads, int(per_pass / (w.batch * w.seqlen * w.headdim))))
    hix = torch.arange(nh, device=inp["x"].device)
    chans = torch.arange(nh * w.headdim, device=inp["x"].device)
    sub = dict(x=inp["x"].index_select(2, chans), dt=inp["dt"].index_select(2, hix),
               A=inp["A"].index_select(0, hix), B=inp["B"], C=inp["C"],
               D=inp["D"].index_select(0, chans), z=inp["z"].index_select(2, chans), h0=None)
    host = {k: (oracle._f64(v) if v is not None else None) for k, v in sub.items()}
    passes, dt = _oracle_passes(lambda: orc.ssd_fwd(**host, headdim=w.headdim), seconds)
    elems = w.batch * w.seqlen * nh * w.headdim * passes
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: all {w.batch} rows x {w.seqlen} tokens x first {nh} of "
                      f"{w.nheads} heads, fp64, {_passes_text(passes, dt)}"}


def conv_bytes(w, state_in):
    """Bytes one convolution call must move: x in and y out (I/O dtype), the
    handed-on state out and, when there is one, the carried state in (I/O
    dtype), weight and bias in (fp32)."""
    s = 4 if w.io == "f32" else 2
    b, l, d, k = w.batch, w.seqlen, w.dim, w.width
    return 2 * b * l * d * s + b * d * k * s * (2 if state_in else 1) + d * k * 4 + d * 4


def gpu_clock_sample(step, max_seconds=2.5):
    """The GFX clock the step runs at, for the record. The GPU's metrics
    table (read through amdsmi) is refreshed by the firmware about once a
    second, so after the timed region the step keeps running, untimed (eight
    steps between readings, the queue drained after each), until the table
    has been refreshed twice while it ran or `max_seconds` pass; the per-XCD
    current GFX clocks of the refreshed tables are reported. Returns None
    when amdsmi is missing, sees more than one GPU or no refresh comes."""
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) != 1:
            return None
        stamp = amdsmi.amdsmi_get_gpu_metrics_info(handles[0]).get("system_clock_counter")
        tables = []
        i = 0
        t_end = time.perf_counter() + max_seconds
        while time.perf_counter() < t_end and len(tables) < 2:
            for _ in range(8):
                step(i)
                i += 1
            m = amdsmi.amdsmi_get_gpu_metrics_info(handles[0])
            if m.get("system_clock_counter") != stamp:
                stamp = m.get("system_clock_counter")
                xcd = [int(c) for c in (m.get("current_gfxclks") or [])
                       if isinstance(c, (int, float)) and c > 0]
                if xcd:
                    tables.append(xcd)
            torch.cuda.synchronize()
        torch.cuda.synchronize()
        if not tables:
            return None
        flat = [c for t in tables for c in t]
        return {"mean_MHz": round(sum(flat) / len(flat)), "min_MHz": min(flat),
                "max_MHz": max(flat), "xcd_MHz_last": tables[-1], "tables": len(tables),
                "how": "amdsmi metrics tables refreshed while the step repeated untimed "
                       "right after the timed region"}
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


# Untimed steps run before the warm-up ones: the GFX clock climbs from idle
# over tens of milliseconds of load, and 50 steps timed after only 5 warm-up
# steps of the Mamba-2.8B layer ran 9% slower (368-374 us) than after 100
# (341 us). Filled in by _spin_up and reported on every bench line.
SPIN_UP = {"seconds": 0.0, "steps": 0}


def _spin_up(step, seconds):
    import torch
    n = 0
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            step(n)
            n += 1
        torch.cuda.synchronize()
    SPIN_UP.update(seconds=seconds, steps=n)
    return n


def _time_steps(step, warmup, steps, stream, spin_up=0.0):
    import torch
    _spin_up(step, spin_up)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0


def bench_conv(args, w):
    """One step = one causal_conv1d_fwd (+ silu) over the whole workload,
    handing on the last W inputs; the convolution kernel and the small
    state kernel are both inside the timed region."""
    import torch

    import selective_state_space_40_amd as ms
    import ssm_workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.load_library()
    sets = [W.generate_conv(w, device=dev, seed=w.seed + 101 * i) for i in range(2)]
    y = torch.empty_like(sets[0]["x"])
    st = torch.empty(w.batch, w.dim, w.width, dtype=y.dtype, device=dev)

    def step(i):
        inp = sets[i % 2]
        ms.conv1d_fwd(inp["x"], inp["weight"], inp["bias"], inp["state_in"], out=y, state_out=st)

    ms_per_step, wall = _time_steps(step, args.warmup, args.steps, torch.cuda.current_stream(dev),
                                      args.spin_up)
    sec = ms_per_step / 1e3
    elems = w.batch * w.seqlen * w.dim
    nbytes = conv_bytes(w, sets[0]["state_in"] is not None)
    gbps = nbytes / sec / 1e9
    cpu = None if args.no_cpu_baseline else cpu_baseline_conv(w, sets[0], args.cpu_seconds)
    clock = gpu_clock_sample(step)
    line = {
        "metric": "short causal convolution elements/s (B*L*D) and achieved HBM GB/s",
        "value": elems / sec, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "dim": w.dim,
                   "width": w.width, "io_dtype": w.io, "silu": True,
                   "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1), "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "conv1d_fwd_kernel + conv1d_state_out_kernel",
                     "algorithmic_bytes": nbytes},
        "gpu_clock": clock,
        "spin_up": dict(SPIN_UP),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_conv_decode(args, w):
    """One step = one causal_conv1d_update per layer over all layers, each
    with its own state, replayed as a HIP graph."""
    import torch

    import selective_state_space_40_amd as ms
    import ssm_workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ms.load_library()
    layers = [W.generate_conv_decode_layer(w, l, device=dev) for l in range(w.layers)]
    ys = [torch.empty_like(L["x"]) for L in layers]

    def run():
        for L, y in zip(layers, ys):
            ms.conv1d_update(L["state"], L["x"], L["weight"], L["bias"], out=y)

    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        run()
    torch.cuda.current_stream(dev).wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    ms_per_step, wall = _time_steps(lambda i: graph.replay(), args.warmup, args.steps,
                                    torch.cuda.current_stream(dev), args.spin_up)
    sec = ms_per_step / 1e3
    s = 4 if w.io == "f32" else 2
    per_layer = (2 * w.batch * w.dim * w.width * s + 2 * w.batch * w.dim * s
                 + w.dim * w.width * 4 + w.dim * 4)
    nbytes = per_layer * w.layers
    gbps = nbytes / sec / 1e9
    clock = gpu_clock_sample(lambda i: graph.replay())
    line = {
        "metric": "convolution decode elements/s (batch*D*layers per step) and achieved HBM GB/s",
        "value": w.batch * w.dim * w.layers / sec, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "width": w.width,
                   "layers": w.layers, "io_dtype": w.io, "parallelism": "single GPU"},
        "achieved_GBps": round(gbps, 1), "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "conv1d_update_kernel (64 launches per step, graph replay)",
                     "algorithmic_bytes": nbytes},
        "gpu_clock": clock,
        "spin_up": dict(SPIN_UP),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_conv(w, inp, seconds):
    """The fp64 oracle's convolution on the host over the whole workload
    (cheap enough to run in full)."""
    import oracle

    orc = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    host = {k: (oracle._f64(v) if v is not None else None) for k, v in inp.items()}
    passes, dt = _oracle_passes(
        lambda: orc.conv1d_fwd(host["x"], host["weight"], host["bias"], host["state_in"]),
        seconds)
    elems = w.batch * w.seqlen * w.dim * passes
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: the whole workload, fp64, {_passes_text(passes, dt)}"}


def cpu_baseline(w, inp, channels, softplus=False, seconds=10.0):
    """The fp64 oracle, as it is, on the host over a channel sample of the
    same workload (all batch rows, all tokens)."""
    import numpy as np
    import torch

    import oracle

    orc = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    if channels <= 0:
        # one pass sized to at most ~`seconds` at ~1e7 elements/s per core
        per_core = 1.0e7
        channels = int(max(seconds, 1.0) * per_core * threads / (w.batch * w.seqlen))
        channels = max(8, min(w.dim, channels))
    idx = torch.arange(channels, device=inp["x"].device)
    sub = {k: v for k, v in dict(
        x=inp["x"].index_select(2, idx), delta=inp["delta"].index_select(2, idx),
        A=inp["A"].index_select(0, idx), B=inp["B"], C=inp["C"], D=inp["D"].index_select(0, idx),
        z=inp["z"].index_select(2, idx), h0=None,
        delta_bias=inp["delta_bias"].index_select(0, idx) if softplus else None).items()}
    host = {k: (oracle._f64(v) if v is not None else None) for k, v in sub.items()}
    passes, dt = _oracle_passes(lambda: orc.scan_fwd(**host, delta_softplus=softplus), seconds)
    elems = w.batch * w.seqlen * channels * passes
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: all {w.batch} batch rows x {w.seqlen} tokens x first "
                      f"{channels} of {w.dim} channels, fp64, {_passes_text(passes, dt)}"}


if __name__ == "__main__":
    main()
