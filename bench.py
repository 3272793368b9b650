"""Benchmark of Sketch Attention compression on one MI355X.

A step is one sa_compress_batch call over one batch of synthetic histories:
fold-free fused pass (affinity, prototype-axis softmax, aggregation) plus the
split-n reduction, i.e. the whole cache-miss path of the SequenceO1 page
(section 2.4) for that batch.  Inputs are resident in HBM before timing
starts; the batch is rotated over several copies whose total size exceeds
the 256 MB Infinity Cache, so X is read from HBM.

Default workload: 4 users x n = 100000 behaviours, d = 128, k = 256
prototypes, bfloat16 inputs with float32 accumulation.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
MALL_BYTES = 256 * 2 ** 20
MEDIAN_STEPS = 50  # steps of the separate per-step pass whose median is reported beside the mean


def kernel_timing_steps(steps: int) -> int:
    """Steps of the kernel-timing pass that follows the timed region: every one
    of its launches records HIP events on its own dispatch (at least 50, and at
    least as many as the timed region).  The timed region carries no events: a
    step whose launches record them costs the GPU several microseconds more."""
    return max(steps, MEDIAN_STEPS)


def timing_period(steps: int) -> int:
    """Kernel durations are taken on every step of a short timed region
    (fewer than 50 steps) and on every 8th step of a long one, where
    event-carrying launches would cost the host enough to starve small batches."""
    return 1 if steps < 50 else 8


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def median_step_us(run, steps: int) -> float:
    """Median over `steps` single steps, each bracketed by events on the launch
    stream (torch's current stream, which is the stream every call uses)."""
    stream = torch.cuda.current_stream()
    times = []
    for i in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run(i)
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    return float(np.median(times))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sketch_attention_amd", "csrc")
METRIC = "history behaviors/sec compressed (n=100K,k=256,d=128); % bf16 MFMA/HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_flops(k: int, d: int, rows: int) -> float:
    """Affinity plus aggregation, 2kd + 2kd per history row (softmax and fold excluded)."""
    return 4.0 * k * d * rows


def algorithmic_bytes(rows: int, users: int, k: int, d: int, elem: int) -> float:
    """X read once plus the float32 sketches written once."""
    return float(rows) * d * elem + 4.0 * users * k * d


def cpu_baseline(wl, budget_s: float, layers=None, norm: str = "prototypes"):
    """Time the fp64 CPU oracle on whole users of the workload, cycling over
    them until about budget_s seconds have passed (the refinement stack's
    oracle when `layers` holds its weights)."""
    from threadpoolctl import threadpool_info

    from oracle import refine_oracle, sa_oracle

    params = None
    if layers is not None:
        params = [refine_oracle.LayerParams(**{k: np.asarray(v, dtype=np.float64) for k, v in lay.items()})
                  for lay in layers]
    rows = 0
    users = 0
    t0 = time.perf_counter()
    while True:
        u = users % wl.num_users
        if norm == "history":
            sa_oracle.history_sketch_user(wl.user_rows(u), wl.P, wl.W_Q, wl.W_K, wl.tau)
        elif params is None:
            sa_oracle.sketch_user(wl.user_rows(u), wl.P, wl.W_Q, wl.W_K, wl.tau)
        else:
            refine_oracle.stack_user(wl.user_rows(u), wl.P, params, wl.tau)
        rows += int(wl.offsets[u + 1] - wl.offsets[u])
        users += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {
        "value": rows / dt if dt > 0 else None,
        "unit": "behaviors/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{users} user {'comparator summaries' if norm == 'history' else 'sketches' if params is None else f'{len(params)}-layer stacks'} cycling over "
                  f"the {wl.num_users} users of the workload ({rows} rows), fp64 numpy/OpenBLAS, {dt:.2f} s",
    }


def fused_kernel_name(dtype: str, d: int, k: int, norm: str = "prototypes") -> str:
    """Name of the fused kernel the library's planner picks for a shape (labels only; the rule of make_plan):
    bf16 d = 128 beyond 512 prototypes runs the two phases on sa_stream32_kernel, bf16 d = 128 with 128 < k <= 256
    the 32x32x16 lanes pass sa_wide_kernel (the comparator keeps sa_stream_kernel), other bf16 with k > 32 the
    streamed sa_stream_kernel, and the rest the lockstep sa_fused_kernel."""
    if dtype != "bf16" or k <= 32:
        return "sa_fused_kernel"
    if norm == "prototypes" and d == 128 and k > 512:
        return "sa_stream32_kernel"
    if norm == "prototypes" and d == 128 and 128 < k <= 256:
        return "sa_wide_kernel"
    return "sa_stream_kernel"


def kernel_source_hash(dtype: str = "bf16", d: int = 128) -> str:
    """sha256 over the sources and compiler options that decide the fused kernel
    a launch runs (include paths left out: they differ between checkouts)."""
    from sketch_attention_amd import build as _build
    names = ["sa_fused.hpp", "sa_stream.hpp", "sa_stream32.hpp", "sa_wide.hpp", f"sa_fused_{dtype}_d{d}.hip", f"sa_stream_d{d}.hip",
             "sa_kernels.hip", "sa_internal.h", "sa_api.cpp"]
    files = [os.path.join(CSRC, f) for f in names if os.path.exists(os.path.join(CSRC, f))]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    flags = [f for f in _build.HIPCC_FLAGS if not f.startswith("-I")]
    h.update(repr((flags, sorted(_build.VGPR_FORM))).encode())
    return h.hexdigest()


def measured_traffic(workload: str, dtype: str, d: int):
    """HBM bytes per fused launch from the committed profiler summary of this
    workload, or None when there is none or the kernel has changed since."""
    path = os.path.join(PROFILES, f"sa_fused_{workload}_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^([a-z0-9_]+): (\S+)$", line.strip())
            if m:
                kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256") != kernel_source_hash(dtype, d):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(steps: int) -> None:
    """Plain elementwise copies of known size (1 GiB read, 1 GiB written per
    dispatch), for scaling the HBM byte counters of a profiler run."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        torch.neg(src, out=dst)   # one vectorised elementwise kernel: read once, write once
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "elementwise neg (float32)", "bytes_read_per_dispatch": nbytes,
                      "bytes_written_per_dispatch": nbytes, "dispatches": steps}), flush=True)


def grad_cpu_baseline(wl, G, budget_s: float):
    """Time the fp64 gradient oracle on whole users, cycling until about budget_s seconds have passed."""
    from threadpoolctl import threadpool_info

    from oracle import grad_oracle

    rows = users = 0
    t0 = time.perf_counter()
    while True:
        u = users % wl.num_users
        grad_oracle.sketch_grad_user(wl.user_rows(u), wl.P, wl.W_Q, wl.W_K, wl.tau, G[u])
        rows += int(wl.offsets[u + 1] - wl.offsets[u])
        users += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": rows / dt if dt > 0 else None, "unit": "behaviors/s", "cores": int(threads), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{users} user gradients cycling over the {wl.num_users} users of the workload ({rows} rows), "
                      f"fp64 numpy/OpenBLAS, {dt:.2f} s"}


def run_grad(args, wl, Xs, copies, offs, dev) -> int:
    """Backward pass: one step = sa_grad_compute over the whole batch.  The
    roofline is that of the longer of the two streamed passes, on its
    algorithmic share: 6kd FLOP per row for the statistics pass (s', dA and
    dQ' = dS X), 4kd for the dX pass (its recomputation of s' and dA, 4kd more
    per row, is not counted)."""
    from sketch_attention_amd import SketchAttentionGrad, binding, workloads

    dt = torch.bfloat16
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)
    G = workloads.make_upstream_grad(wl.num_users, wl.k, wl.d, seed=0)
    Gd = torch.from_numpy(G).to(dev)
    h = SketchAttentionGrad(t(wl.P), t(wl.W_Q), t(wl.W_K), wl.tau)
    gX = torch.empty_like(Xs[0])
    gP = torch.empty((wl.k, wl.d), dtype=torch.float32, device=dev)
    gQ = torch.empty((wl.d, wl.d), dtype=torch.float32, device=dev)
    gK = torch.empty_like(gQ)
    stream = torch.cuda.current_stream(dev)
    run = lambda i: binding.sa_grad_compute(h.handle, Xs[i % copies], offs, Gd, gX, gP, gQ, gK, stream)
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize(dev)
    binding.sa_grad_read_kernel_timing(h.handle)
    t0 = time.perf_counter()
    period = timing_period(args.steps)
    for i in range(args.steps):
        timed = i % period == 0
        if timed:
            binding.sa_grad_set_kernel_timing(h.handle, True)
        run(i)
        if timed:
            binding.sa_grad_set_kernel_timing(h.handle, False)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    stats_ms, dx_ms, calls = binding.sa_grad_read_kernel_timing(h.handle)
    h.close()
    ms_per_step = elapsed * 1e3 / args.steps
    n, k, d = wl.total_rows, wl.k, wl.d
    st_us, dx_us = stats_ms * 1e3 / max(calls, 1), dx_ms * 1e3 / max(calls, 1)
    st_tf = 6.0 * k * d * n / (st_us * 1e-6) / 1e12 if st_us > 0 else 0.0
    dx_tf = 4.0 * k * d * n / (dx_us * 1e-6) / 1e12 if dx_us > 0 else 0.0
    log(f"[bench] grad: statistics pass {st_us:.2f} us ({st_tf:.1f} TFLOP/s algorithmic), dX pass {dx_us:.2f} us "
        f"({dx_tf:.1f} TFLOP/s algorithmic, {2 * dx_tf:.1f} executed); whole step {ms_per_step * 1e3:.2f} us "
        f"({10.0 * k * d * n / (ms_per_step * 1e-3) / 1e12:.1f} TFLOP/s over the 10kd FLOP per row)")
    name, us, tf = ("grad_dx_kernel", dx_us, dx_tf) if dx_us >= st_us else ("grad_stats_kernel", st_us, st_tf)
    roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": name, "kernel_avg_us": round(us, 2)}
    cpu = None if args.no_cpu_baseline else grad_cpu_baseline(wl, G, args.cpu_budget)
    if cpu:
        log(f"[bench] cpu baseline: {cpu}")
    line = {
        "metric": "history behaviors/sec through the backward pass (gradients w.r.t. X, P, W_Q, W_K)",
        "value": round(n * args.steps / elapsed, 1), "unit": "behaviors/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.num_users} users x n={n // max(wl.num_users, 1)}, d={d}, k={k}, "
                               f"{wl.dtype}, backward", "users": wl.num_users, "rows": n, "d": d, "k": k,
                   "pass": "backward", "parallelism": "single-gpu"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def action_cpu_baseline(inp, wl, budget_s: float):
    """Time the fp64 oracles (action fusion, then the sketch) on whole users, cycling until about budget_s."""
    from threadpoolctl import threadpool_info

    from oracle import action_oracle, sa_oracle

    rows = users = 0
    t0 = time.perf_counter()
    while True:
        u = users % wl.num_users
        a, b = int(wl.offsets[u]), int(wl.offsets[u + 1])
        x = action_oracle.action_fuse(inp["E"][a:b], inp["actions"][a:b], inp["table"], inp["W_gate"], inp["W_up"],
                                      inp["W_down"])
        sa_oracle.sketch_user(x, wl.P, wl.W_Q, wl.W_K, wl.tau)
        rows += b - a
        users += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": rows / dt if dt > 0 else None, "unit": "behaviors/s", "cores": int(threads), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{users} users (action fusion + sketch) cycling over the {wl.num_users} users of the workload "
                      f"({rows} rows), fp64 numpy/OpenBLAS, {dt:.2f} s"}


def run_actions(args, wl, dev) -> int:
    """One step = the action fusion over every row followed by one compression
    of the rows.  --action-path two-pass: the fusion pass writes X to HBM and
    the sketch pass reads it (two launches); the roofline is the fusion
    pass's, on 2 (2 (d + d_a) d_ff + d_ff d) FLOP per row.  fused: one kernel
    forms the rows in LDS and sketches them (X never written); its roofline
    is on those FLOP plus the sketch's 4 k d per row."""
    from sketch_attention_amd import ActionFusion, SketchAttention, binding, workloads

    d, d_a, d_ff, n_act = wl.d, args.d_a, args.d_ff or 2 * wl.d, args.n_actions
    inp = workloads.make_action_inputs(wl.total_rows, d, d_a, d_ff, n_act, seed=1)
    t = lambda a, dt=torch.bfloat16: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)
    e_bytes = wl.total_rows * d * 2
    copies = max(1, math.ceil(2 * MALL_BYTES / max(e_bytes, 1)) + 1) if e_bytes < 2 * MALL_BYTES else 1
    Es = [t(inp["E"])]
    Es += [Es[0].clone() for _ in range(copies - 1)]
    acts = t(inp["actions"], torch.int32)
    X = torch.empty_like(Es[0])
    af = ActionFusion(t(inp["table"]) if d_a else None, t(inp["W_gate"]), t(inp["W_up"]), t(inp["W_down"]), n_act)
    sa = SketchAttention(t(wl.P), t(wl.W_Q), t(wl.W_K), wl.tau)
    out = torch.empty((wl.num_users, wl.k, d), dtype=torch.float32, device=dev)
    offs = np.ascontiguousarray(wl.offsets, dtype=np.int64)
    stream = torch.cuda.current_stream(dev)

    fused = args.action_path == "fused"

    def step(i):
        if fused:
            binding.sa_action_compress_batch(af.handle, sa.handle, Es[i % copies], acts, offs, out, stream)
        else:
            binding.sa_action_fuse(af.handle, Es[i % copies], acts, X, stream)
            binding.sa_compress_batch(sa.handle, X, offs, out, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)
    binding.sa_action_read_kernel_timing(af.handle)
    binding.sa_read_kernel_timing(sa.handle)
    t0 = time.perf_counter()
    period = timing_period(args.steps)
    for i in range(args.steps):
        timed = i % period == 0
        if timed:
            binding.sa_action_set_kernel_timing(af.handle, True)
            binding.sa_set_kernel_timing(sa.handle, True)
        step(i)
        if timed:
            binding.sa_action_set_kernel_timing(af.handle, False)
            binding.sa_set_kernel_timing(sa.handle, False)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    a_ms, a_n = binding.sa_action_read_kernel_timing(af.handle)
    f_ms, _, f_n = binding.sa_read_kernel_timing(sa.handle)
    af.close()
    sa.close()
    n = wl.total_rows
    a_us, f_us = a_ms * 1e3 / max(a_n, 1), f_ms * 1e3 / max(f_n, 1)
    a_flop = 2.0 * (2.0 * (d + d_a) * d_ff + d_ff * d) * n
    ms_per_step = elapsed * 1e3 / args.steps
    if fused:
        flop = a_flop + 4.0 * wl.k * d * n
        tf = flop / (f_us * 1e-6) / 1e12 if f_us > 0 else 0.0
        log(f"[bench] actions (fused prologue): action + sketch kernel {f_us:.2f} us ({tf:.1f} TFLOP/s on the FFN and "
            f"sketch FLOP); whole step {ms_per_step * 1e3:.2f} us (d_a={d_a}, d_ff={d_ff}, {n_act} action types)")
        kern, k_us = "action_sa_kernel", f_us
    else:
        tf = a_flop / (a_us * 1e-6) / 1e12 if a_us > 0 else 0.0
        log(f"[bench] actions: fusion pass {a_us:.2f} us ({tf:.1f} TFLOP/s), fused SA pass {f_us:.2f} us; whole step "
            f"{ms_per_step * 1e3:.2f} us (d_a={d_a}, d_ff={d_ff}, {n_act} action types)")
        kern, k_us = "action_fuse_kernel", a_us
    roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": kern,
            "kernel_avg_us": round(k_us, 2)}
    cpu = None if args.no_cpu_baseline else action_cpu_baseline(inp, wl, args.cpu_budget)
    if cpu:
        log(f"[bench] cpu baseline: {cpu}")
    line = {
        "metric": "history behaviors/sec through the action fusion and the compression",
        "value": round(n * args.steps / elapsed, 1), "unit": "behaviors/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.num_users} users x n={n // max(wl.num_users, 1)}, d={d}, k={wl.k}, "
                               f"{wl.dtype}, action fusion d_a={d_a} d_ff={d_ff} ({args.action_path})",
                   "users": wl.num_users, "rows": n, "action_path": args.action_path,
                   "d": d, "k": wl.k, "d_a": d_a, "d_ff": d_ff, "n_actions": n_act, "parallelism": "single-gpu"},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long", choices=["tiny", "recent", "long", "many_proto", "ragged", "final"])
    ap.add_argument("--users", type=int, default=None, help="change the number of users (same per-user shape)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the on-device ceiling measurements")
    ap.add_argument("--copy-calibration", action="store_true", help="run plain copies only (counter scaling)")
    ap.add_argument("--layers", type=int, default=0,
                    help="run the stacked refinement with this many layers (0: the single SA pass)")
    ap.add_argument("--d-ff", type=int, default=None,
                    help="FFN width of the refinement stack (default 4 d) or of the action fusion (default 2 d)")
    ap.add_argument("--actions", action="store_true",
                    help="build the rows by the action fusion (x = e + SwiGLU-FFN([e; a])) before each compression")
    ap.add_argument("--d-a", type=int, default=64, help="action embedding width for --actions")
    ap.add_argument("--action-path", choices=["two-pass", "fused"], default="two-pass",
                    help="--actions: X through HBM between two passes, or formed inside the sketch kernel")
    ap.add_argument("--n-actions", type=int, default=8, help="action types for --actions")
    ap.add_argument("--grad", action="store_true",
                    help="time the backward pass (gradients w.r.t. X, P, W_Q, W_K) instead of the compression")
    ap.add_argument("--norm", default="prototypes", choices=["prototypes", "history"],
                    help="softmax axis: prototypes (Sketch Attention) or history (the comparator)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2
    conflict = None
    if args.norm == "history" and args.layers:
        conflict = "--norm history runs the single pass only"
    elif args.actions and (args.layers or args.norm != "prototypes" or args.grad):
        conflict = "--actions times the action fusion plus the single pass only"
    elif args.grad and (args.layers or args.norm != "prototypes"):
        conflict = "--grad times the single pass's backward only"
    if conflict:
        print(conflict, file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration(max(args.steps, 1))
        return 0

    from sketch_attention_amd import SketchAttention, binding
    from sketch_attention_amd import workloads

    t_gen = time.perf_counter()
    wl = workloads.named_workload(args.workload, users=args.users)
    log(f"[bench] workload {wl.name}: {wl.recipe}; users={wl.num_users} rows={wl.total_rows} "
        f"(generated in {time.perf_counter() - t_gen:.1f} s)")
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    elem = 2 if wl.dtype == "bf16" else 4
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)
    X0 = t(wl.X)
    x_bytes = wl.total_rows * wl.d * elem
    copies = max(1, math.ceil(2 * MALL_BYTES / max(x_bytes, 1)) + 1) if x_bytes < 2 * MALL_BYTES else 1
    Xs = [X0] + [X0.clone() for _ in range(copies - 1)]
    if args.actions:
        return run_actions(args, wl, dev)
    if args.grad:
        return run_grad(args, wl, Xs, copies, np.ascontiguousarray(wl.offsets, dtype=np.int64), dev)
    sa = SketchAttention(t(wl.P), t(wl.W_Q), t(wl.W_K), wl.tau, norm=args.norm)
    outs = [torch.empty((wl.num_users, wl.k, wl.d), dtype=torch.float32, device=dev) for _ in range(2)]
    offs = np.ascontiguousarray(wl.offsets, dtype=np.int64)
    plan = sa.plan(wl.total_rows)
    log(f"[bench] plan {plan}; input copies {copies} x {x_bytes / 1e6:.1f} MB")
    stream = torch.cuda.current_stream(dev)
    stack_layers = None
    passes = 1  # fused SA passes per step
    if args.layers > 0:
        from sketch_attention_amd import SketchStack
        d_ff = args.d_ff or 4 * wl.d
        stack_layers = workloads.make_stack_layers(d=wl.d, d_ff=d_ff, layers=args.layers, dtype=wl.dtype, seed=11)
        lt = [{n: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt if n in ("W_Q", "W_K") else torch.float32)
               for n, a in lay.items()} for lay in stack_layers]
        stack = SketchStack(t(wl.P), lt, wl.tau)
        passes = args.layers
        log(f"[bench] refinement stack: {args.layers} layers, FFN width {d_ff}")
        handle, bind = stack.handle, binding.sa_stack_compress_batch_bound
        set_timing, read_timing = binding.sa_stack_set_kernel_timing, binding.sa_stack_read_kernel_timing
    else:
        handle, bind = sa.handle, binding.sa_compress_batch_bound
        set_timing, read_timing = binding.sa_set_kernel_timing, binding.sa_read_kernel_timing
    # every (input copy, output) pair's call checked once up front: the timed loop
    # then re-issues C calls only, so the host keeps ahead of the GPU
    calls = {(c, o): bind(handle, Xs[c], offs, outs[o], stream) for c in range(copies) for o in range(2)}

    def compress(i: int) -> None:
        calls[(i % copies, i % 2)]()

    # the device ceilings are measured before the warmup: their loops also bring
    # the chip out of its idle clock state, so a short timed region is not spent
    # on that ramp
    ceil = None
    if not args.no_ceilings:
        ceil = measured_ceilings()
        log(f"[bench] ceilings: {ceil}")

    for i in range(args.warmup):
        compress(i)
    torch.cuda.synchronize(dev)
    read_timing(handle)  # discard anything recorded so far

    # the timed region: exactly `steps` steps bracketed by synchronisations, no events
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        compress(i)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {elapsed * 1e3:.2f} ms")

    # kernel durations: a pass of the same steps right after, each launch recording
    # HIP events on its own dispatch (on the launch stream)
    timed_steps = kernel_timing_steps(args.steps)
    set_timing(handle, True)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    for i in range(timed_steps):
        compress(args.steps + i)
    set_timing(handle, False)
    torch.cuda.synchronize(dev)
    timing_wall = time.perf_counter() - t1
    fused_ms, reduce_ms, launches = read_timing(handle)
    log(f"[bench] kernel timing over {timed_steps} further steps ({launches} fused launches; "
        f"{timing_wall * 1e6 / timed_steps:.2f} us per step by wall clock in that pass)")

    ms_per_step = elapsed * 1e3 / args.steps
    value = wl.total_rows * args.steps / elapsed
    flops = algorithmic_flops(wl.k, wl.d, wl.total_rows)
    nbytes = algorithmic_bytes(wl.total_rows, wl.num_users, wl.k, wl.d, elem)
    fused_avg_ms = fused_ms / max(launches, 1)
    # launches == timed steps unless the batch spans several launches; per-launch work
    per_launch_flops = flops * passes * timed_steps / max(launches, 1)
    per_launch_bytes = nbytes * passes * timed_steps / max(launches, 1)
    mfma_peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    tflops = per_launch_flops / (fused_avg_ms * 1e-3) / 1e12 if fused_avg_ms > 0 else 0.0
    gbs = per_launch_bytes / (fused_avg_ms * 1e-3) / 1e9 if fused_avg_ms > 0 else 0.0
    ridge = mfma_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if flops / nbytes >= ridge else "hbm"
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(tflops / mfma_peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    roof["traffic"] = measured_traffic(wl.name, wl.dtype, wl.d) if (args.users is None and not args.layers and
                                                                     args.norm == "prototypes") else None
    roof["kernel"] = fused_kernel_name(wl.dtype, wl.d, wl.k, args.norm)
    roof["kernel_avg_us"] = round(fused_avg_ms * 1e3, 2)
    roof["kernel_launches_timed"] = int(launches)
    log(f"[bench] fused kernel avg {fused_avg_ms * 1e3:.2f} us ({tflops:.1f} TFLOP/s, {gbs:.0f} GB/s), "
        f"reduce avg {reduce_ms / max(launches, 1) * 1e3:.2f} us; whole step {ms_per_step * 1e3:.2f} us "
        f"({flops * passes / (ms_per_step * 1e-3) / 1e12:.1f} TFLOP/s in the SA passes)")

    med_us = median_step_us(compress, max(MEDIAN_STEPS, args.steps))
    log(f"[bench] median of {max(MEDIAN_STEPS, args.steps)} single steps: {med_us:.2f} us")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_budget, stack_layers, args.norm)
        log(f"[bench] cpu baseline: {cpu}")

    sa.close()
    if args.layers > 0:
        stack.close()
    line = {
        "metric": (METRIC if args.norm == "prototypes" else "history behaviors/sec summarised by the history-axis "
                   "softmax comparator") if not args.layers
        else f"history behaviors/sec through a {args.layers}-layer refinement stack",
        "value": round(value, 1),
        "unit": "behaviors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "median_step_us": round(med_us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.num_users} users x n={wl.total_rows // max(wl.num_users, 1)}, "
                        f"d={wl.d}, k={wl.k}, {wl.dtype}",
            "users": wl.num_users,
            "rows": wl.total_rows,
            "d": wl.d,
            "k": wl.k,
            **({"layers": args.layers, "d_ff": args.d_ff or 4 * wl.d} if args.layers else {}),
            **({"norm": "history"} if args.norm == "history" else {}),
            "parallelism": "single-gpu",
        },
        "roofline": roof,
        "ceilings": ceil,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def measured_ceilings() -> dict:
    """On-device ceilings beside the published peaks (the fractions in
    `roofline` stay against the published ones)."""
    from sketch_attention_amd import binding
    c = binding.sa_measure_ceilings()
    read_gbs = binding.sa_measure_hbm_read()
    return {
        "mfma_bf16_16x16x32_tflops": round(c["mfma_bf16_tflops"], 1),
        "mfma_bf16_32x32x16_tflops": round(c["mfma_bf16_32x32_tflops"], 1), "mfma_bf16_spec_tflops": PEAK_BF16_TFLOPS,
        "hbm_copy_gbs": round(c["copy_gbs"], 1), "hbm_read_gbs": round(read_gbs, 1), "hbm_spec_gbs": PEAK_HBM_GBS,
        "valu_fp32_fma_tflops": round(c["valu_fma_tflops"], 1), "valu_fp32_spec_tflops": 157.3,
        "exp2_per_sec": float(f"{c['exp2_per_sec']:.4g}"),
        "how": "bf16 matrix-core loops of 16x16x32 and of 32x32x16 products; fp32 FMA and hardware exp2 loops of independent chains; "
               "streaming copy of 1 GiB (read + write counted); read-only stream of 1 GiB",
    }


if __name__ == "__main__":
    sys.exit(main())
