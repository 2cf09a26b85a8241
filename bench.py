#!/usr/bin/env python3
"""Benchmark of the LoReS quantized recurrent-state decode step on one MI355X.

A step is one decode step of the whole batch: every (sequence, head) state is
dequantized, updated, read out and requantized in place.  Inputs for all
timed steps are generated on the device before timing.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C5]

Workloads (synthetic, shapes of the decode layers the method targets):
  C5 (default) large batch, B=2048 H=32 d=128, 16 int8 + 16 int4 heads (the
     largest workload: its 839 MB state exceeds the 256 MB last-level cache,
     so its bytes are HBM bytes)
  C2 Gated-DeltaNet decode, B=64 H=32 d_k=d_v=128, bf16 q/k/v, int8 state
  C3 Mamba-2 / SSD decode, B=256 H=128 d_v=64 d_k=128, no delta correction, int8
  C4 KDA per-channel decay, B=128 H=32 d=128, 8 bf16 + 24 int8 heads
  C5i6 the same shape with the slowest half of the heads in int6 (5.25 bits)
  C1 is the tiny parity case (launch-bound; not a throughput workload).
--mode copy times a plain device copy (the HBM calibration used for the
rocprofv3 byte counters); --mode error runs the error-accumulation harness
(quantized state against an fp32 twin over a long horizon) and prints its
report instead; --mode sweep times the step kernel per state precision at the
large-batch shape (which classes are HBM-bound and which VALU-bound).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "state-updates/s (B*H*steps) and achieved HBM GB/s vs peak, quantized decode"
HBM_PEAK_GBPS = 8000.0
CSRC = os.path.join(ROOT, "quantized_linear_recurrence_amd", "csrc")


def _code_only(text):
    """C++ source without comments and blank space, so that a comment edit
    leaves the hash alone."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the step kernel's code (its header and every step translation
    unit, comments dropped): a stored HBM byte count is used only while it
    matches."""
    h = hashlib.sha256()
    names = sorted(f for f in os.listdir(CSRC) if f.startswith("lores_step") or f == "lores_internal.h")
    for f in names:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def unit_bytes(prec, dk, dv, in_bytes, per_channel, key=False, window=1):
    """Algorithmic bytes of one state update: the state read and written once,
    plus q, k, v, alpha, beta read and o written.  The scales are one fp32 per
    value row, or per key column with key=True.  A windowed state (window W >
    1, scaled classes) is read every step and written once per window, and
    per window its buffer is written once and read back by the later steps
    of the window (token tau is read by the W - tau later steps): averaged
    per step, state (1 + 1/W) + buffer ((W - 1) + W (W - 1) / 2) / W slots of
    (d_v + d_k + 1) fp32 (d_v + 2 d_k with a decay per key channel)."""
    ns = dk if key else dv
    state = {0: 4 * dv * dk, 1: 2 * dv * dk, 2: dv * dk + 4 * ns, 3: dv * dk // 2 + 4 * ns,
             4: 6 * dv * dk // 8 + 4 * ns, 5: dv * dk + 4 * ns}[prec]
    io = 2 * dk * in_bytes + dv * in_bytes + (4 * dk if per_channel else 4) + 4 + 4 * dv
    if window > 1 and prec in (2, 3, 4, 5):
        W = window
        slot = 4 * (dv + dk + (dk if per_channel else 1))
        return state * (W + 1) / W + slot * ((W - 1) + W * (W - 1) / 2) / W + io
    return 2 * state + io


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="C5", choices=["C1", "C2", "C3", "C4", "C5", "C5i6"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target time of the oracle baseline sample (per worker process)")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="worker processes of the oracle baseline (at most the host's cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy", "error", "sweep"])
    ap.add_argument("--sweep-only", default="",
                    help="--mode sweep: only the rows whose label contains this text")
    ap.add_argument("--error-steps", type=int, default=2048,
                    help="horizon of the error-accumulation harness (--mode error)")
    ap.add_argument("--copy-mib", type=int, default=2048)
    ap.add_argument("--repeats", type=int, default=5,
                    help="repetitions of the K timed steps after the timed region, from a fresh "
                         "state each, reported as their median, min and max")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="how the timed steps are issued")
    ap.add_argument("--state", default="assigned",
                    choices=["assigned", "fp32", "bf16", "int8", "int4", "int6", "fp8"],
                    help="precision of every head: the workload's decay-based assignment "
                         "(default), or one precision for all heads (fp32 / bf16: the "
                         "unquantized-state comparison)")
    ap.add_argument("--window", type=int, default=1,
                    help="requantize the int / fp8 heads once per window of this many steps "
                         "(windowed states; 1: every step)")
    ap.add_argument("--scale-axis", default="value", choices=["value", "key"],
                    help="scale grouping of the int / fp8 heads: one scale per value row "
                         "(the method's choice) or per key column")
    return ap.parse_args(argv)


def effective_bits(head_prec, dk, dv, key=False):
    """Mean stored bits per state element: codes plus the fp32 scales."""
    per = []
    for p in head_prec:
        bits = {0: 32, 1: 16, 2: 8, 3: 4, 4: 6, 5: 8}[p]
        if p in (2, 3, 4, 5):
            bits += 32.0 * (dk if key else dv) / (dk * dv)
        per.append(bits)
    return sum(per) / len(per)


def copy_reference(torch, nbytes):
    """Event time of a plain device-to-device copy that reads and writes
    nbytes / 2 each (the state's read + write traffic), after a warm copy."""
    n = max(int(nbytes) // 2, 1)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    return {"bytes": 2 * n, "us": us, "GBps": 2 * n / us / 1e3}


def copy_mode(args, torch):
    """Plain device-to-device copy of --copy-mib MiB, 10 times: the calibration
    kernel for FETCH_SIZE / WRITE_SIZE counters and a measured copy bandwidth."""
    n = args.copy_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "ms_per_copy": ms, "copy_GBps": 2 * n / ms / 1e6}), flush=True)


SWEEP = [  # (label, B, H, d_k, d_v, per-head precision, delta[, "key"][, window])
    ("int8+int4 (C5)", 2048, 32, 128, 128, [2] * 16 + [3] * 16, 1),
    ("int8+int4 (C5), delta 0", 2048, 32, 128, 128, [2] * 16 + [3] * 16, 0),
    ("int8", 2048, 32, 128, 128, [2] * 32, 1),
    ("int8, delta 0", 2048, 32, 128, 128, [2] * 32, 0),
    ("int6", 2048, 32, 128, 128, [4] * 32, 1),
    ("fp8 (E4M3)", 2048, 32, 128, 128, [5] * 32, 1),
    ("int4", 2048, 32, 128, 128, [3] * 32, 1),
    ("int4, delta 0", 2048, 32, 128, 128, [3] * 32, 0),
    ("bf16", 1024, 32, 128, 128, [1] * 32, 1),
    ("int8, d_v 64 (C3 shape), delta 0", 256, 128, 128, 64, [2] * 128, 0),
    ("int8, key columns", 2048, 32, 128, 128, [2] * 32, 1, "key"),
    ("int4, key columns", 2048, 32, 128, 128, [3] * 32, 1, "key"),
    ("int6, key columns", 2048, 32, 128, 128, [4] * 32, 1, "key"),
    ("fp8 (E4M3), key columns", 2048, 32, 128, 128, [5] * 32, 1, "key"),
    ("int8, d_v 64 (C3 shape), key columns", 256, 128, 128, 64, [2] * 128, 0, "key"),
    ("int8, window 4", 2048, 32, 128, 128, [2] * 32, 1, 4),
    ("int8, window 8", 2048, 32, 128, 128, [2] * 32, 1, 8),
    ("int4, window 8", 2048, 32, 128, 128, [3] * 32, 1, 8),
    ("int8+int4 (C5), window 8", 2048, 32, 128, 128, [2] * 16 + [3] * 16, 1, 8),
    ("int8+int4 (C5), key columns, window 4", 2048, 32, 128, 128, [2] * 16 + [3] * 16, 1, "key", 4),
    ("int8, d_k 256 (split rows)", 1024, 32, 256, 128, [2] * 32, 1),
    ("int4, d_k 256 (split rows)", 1024, 32, 256, 128, [3] * 32, 1),
    ("int8+int4, d_k 256 (split rows, fused pair)", 1024, 32, 256, 128, [2] * 16 + [3] * 16, 1),
    ("int8, d_k 256, key columns", 1024, 32, 256, 128, [2] * 32, 1, "key"),
    ("bf16, d_k 256 (split rows)", 512, 32, 256, 128, [1] * 32, 1),
    ("bf16+int8, d_k 256 (split rows, side by side)", 1024, 32, 256, 128, [1] * 8 + [2] * 24, 1),
]


def sweep_mode(args, torch):
    """Achieved HBM throughput of the step kernel per state precision at the
    large-batch shape: which classes sit on the HBM roof and which on the
    VALU roof.  Random unit-norm q, k; v ~ N(0, 1); alpha in [0.7, 1);
    fp32 inputs; 64 steps in a captured graph after 8 warm-up steps."""
    import quantized_linear_recurrence_amd as lores
    dev = torch.device("cuda:0")
    rows = []
    for label, B, H, dk, dv, prec, delta, *ax in SWEEP:
        if args.sweep_only and args.sweep_only not in label:
            continue
        key = "key" in ax
        window = next((a for a in ax if isinstance(a, int)), 1)
        g = torch.Generator(device=dev)
        g.manual_seed(args.seed)

        def unit(x):
            return x / x.norm(dim=-1, keepdim=True)
        q = unit(torch.randn(B, H, dk, generator=g, device=dev))
        k = unit(torch.randn(B, H, dk, generator=g, device=dev))
        v = torch.randn(B, H, dv, generator=g, device=dev)
        alpha = (0.7 + 0.3 * torch.rand(B, H, generator=g, device=dev)).contiguous()
        beta = (2 * torch.sigmoid(torch.randn(B, H, generator=g, device=dev))).contiguous()
        st = lores.lores_state_alloc(B, H, dk, dv, prec, device=dev,
                                     scale_axis=lores.LORES_SCALE_KEY if key else 0, window=window)
        o = torch.empty(B, H, dv, device=dev)
        for t in range(1, 9):
            lores.lores_decode_step(st, q, k, v, alpha, beta, delta, args.seed, t, o=o)
        steps = 64                        # a whole number of windows: each replay starts one
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for t in range(9, 9 + steps):
                lores.lores_decode_step(st, q, k, v, alpha, beta, delta, args.seed, t, o=o)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        nbytes = sum(B * prec.count(c) * unit_bytes(c, dk, dv, 4, False, key, window)
                     for c in range(6))
        gbs = nbytes / us / 1e3
        rows.append({"state": label, "B": B, "H": H, "d_k": dk, "d_v": dv, "delta": delta,
                     "scale_axis": "key" if key else "value", "window": window,
                     "us_per_step": us, "updates_per_s": B * H / (us * 1e-6), "GBps": gbs,
                     "frac": gbs / HBM_PEAK_GBPS})
        print(f"[sweep] {label:34s} {us:8.1f} us/step {gbs:7.0f} GB/s  {gbs / HBM_PEAK_GBPS:.3f}",
              file=sys.stderr, flush=True)
    print(json.dumps({"mode": "sweep", "rows": rows}), flush=True)


def _oracle_worker(job):
    """One CPU worker of the baseline (a child process): the oracle, as it
    stands, stepping its own (sequence, head) units from the common start time
    until target_s has passed.  Returns (updates, start, end) wall times."""
    import numpy as np
    from oracle import step as ostep
    from oracle import window as owin
    try:                                   # one thread per worker: BLAS pools stay at 1
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass
    units, host, head_prec, dims, target_s, seed, axis, window, t_start = job
    dk, dv, delta = dims
    by_class = {}
    for i, (b, h) in enumerate(units):
        by_class.setdefault(head_prec[h], []).append((i, b, h))
    states = {c: ostep.zero_state(c, len(us), dv, dk, axis=axis) for c, us in by_class.items()}
    bufs = {c: owin.empty_buffer(len(us), window, dv, dk) for c, us in by_class.items()}
    while time.time() < t_start:
        time.sleep(0.001)
    t0 = time.time()
    steps = 0
    while True:
        xin = host[steps % len(host)]
        for c, us in by_class.items():
            rows = np.array([i for i, _, _ in us])
            bs = np.array([b for _, b, _ in us])
            hs = np.array([h for _, _, h in us])
            a = tuple(xin[k][rows] for k in ("q", "k", "v", "alpha", "beta"))
            if window > 1 and c in ostep.SCALED:
                states[c], bufs[c], _ = owin.window_step(c, states[c], bufs[c], *a, delta, seed,
                                                         steps + 1, bs, hs, window)
            else:
                states[c], _ = ostep.decode_step(c, states[c], *a, delta, seed, steps + 1, bs,
                                                 hs, axis=axis)
        steps += 1
        if time.time() - t0 >= target_s:
            break
    return len(units) * steps, t0, time.time(), steps


def cpu_baseline(w, inputs, head_prec, target_s, seed, axis="value", window=1, workers=None):
    """Time the oracle (as it stands) on a bounded sample of the same workload,
    on the host's cores: independent worker processes, each stepping its own
    64 (sequence, head) units of the batch (the first units in order), all
    from one common start time for about target_s seconds.  The rate is the
    total state updates over the span from that start to the last worker's
    end.  Windowed states (window > 1) run the oracle's windowed step."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    avail = len(os.sched_getaffinity(0))
    n_workers = max(1, min(workers or 16, avail))
    per = 64
    n_units = min(w.B * w.H, per * n_workers)
    n_workers = -(-n_units // per)
    units = [(u // w.H, u % w.H) for u in range(n_units)]
    T_in = min(inputs["k"].shape[0], 64)
    b_hi = max(b for b, _ in units) + 1
    # the sampled sequences' inputs on the host, [T][unit] per tensor
    host_all = {k: v[:T_in, :b_hi].float().cpu().numpy() for k, v in inputs.items()}
    jobs = []
    t_start = time.time() + 10.0            # the workers' interpreters start meanwhile
    for j in range(n_workers):
        us = units[j * per:(j + 1) * per]
        bs = [b for b, _ in us]
        hs = [h for _, h in us]
        host = [{k: v[t][bs, hs] for k, v in host_all.items()} for t in range(T_in)]
        jobs.append((us, host, list(head_prec), (w.dk, w.dv, w.delta), target_s, seed, axis,
                     window, t_start))
    # fresh interpreters (spawn): the workers never touch the GPU runtime of
    # this process; a worker that fails raises here instead of being restarted
    with ProcessPoolExecutor(n_workers, mp_context=mp.get_context("spawn")) as pool:
        res = list(pool.map(_oracle_worker, jobs))
    updates = sum(r[0] for r in res)
    span = max(r[2] for r in res) - min(r[1] for r in res)
    steps = min(r[3] for r in res)
    return {"value": updates / span, "unit": "state-updates/s", "cores": n_workers,
            "kind": "oracle", "host_cores_available": avail, "blas_threads": 1,
            "sample": f"{n_units} (sequence, head) units of {w.key} ({w.name}), in {n_workers} "
                      f"worker processes of {per} units, >= {steps} decode steps each over "
                      f"{span:.1f} s (NumPy oracle, one thread per process, fp32-exact rounding "
                      f"emulation)"}


def load_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# VALU peak in lane-instructions per second: 256 CUs, each issuing one
# 64-lane VALU instruction per cycle (four SIMD16 units, four cycles per
# wave64 instruction), at 2.4 GHz
VALU_PEAK_LANE_OPS = 256 * 64 * 2.4e9


def load_valu(workload):
    """VALU wave-instructions per launch (SQ_INSTS_VALU) from the committed
    rocprofv3 --pmc summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"valu_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("valu_insts_per_launch")


def limiter(frac_hbm, frac_valu):
    """Which roof the launch sits closer to: "hbm", "valu", or both when the two
    fractions are within 0.05 of each other."""
    if frac_valu is None:
        return "hbm (VALU not profiled on these kernel sources)"
    if abs(frac_hbm - frac_valu) < 0.05:
        return "hbm and valu"
    return "hbm" if frac_hbm > frac_valu else "valu"


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the decode step exchanges nothing between GPUs, so a sharded run is this "
              "single-GPU step on each GPU's share of sequences or heads, and multi-GPU "
              "runs are not supported here.", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    if args.mode == "copy":
        copy_mode(args, torch)
        return
    if args.mode == "sweep":
        sweep_mode(args, torch)
        return
    if args.mode == "error":
        from quantized_linear_recurrence_amd import error_harness
        t0 = time.perf_counter()
        rows = error_harness.run_suite(T=args.error_steps, seed=args.seed)
        print(json.dumps({"mode": "error", "metric": "relative state error vs an fp32 twin",
                          "T": args.error_steps, "B": 32, "H": 12, "d_k": 128, "d_v": 128,
                          "delta": 0, "inputs": "random unit k, q; random v; beta 0.5",
                          "seconds": time.perf_counter() - t0, "results": rows}), flush=True)
        return

    import quantized_linear_recurrence_amd as lores
    from workloads import get_workload, make_inputs

    w = get_workload(args.workload)
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    win = args.window
    if win > 1:
        K, W = -(-K // win) * win, -(-W // win) * win       # whole windows
    T_in = min(w.T, max(K, W, 1))
    print(f"[bench] generating {T_in} steps of {w.key} inputs on {dev}", file=sys.stderr, flush=True)
    inputs = make_inputs(w, args.seed, dev, T=T_in)

    # precision per head from the decay statistic of a calibration sample
    if args.state != "assigned":
        code = {"fp32": 0, "bf16": 1, "int8": 2, "int4": 3, "int6": 4, "fp8": 5}[args.state]
        head_prec = [code] * w.H
    elif len(w.tiers) == 1:
        head_prec = [w.tiers[0][1]] * w.H
    else:
        cal = inputs["alpha"][:min(T_in, 32)].float().cpu().numpy()
        cal = cal.reshape(cal.shape[0] * cal.shape[1], w.H, -1)
        head_prec = lores.lores_assign_precision(lores.lores_decay_stat(cal),
                                                 [f for f, _ in w.tiers], [p for _, p in w.tiers])

    in_bytes = 2 if w.in_bf16 else 4
    key = args.scale_axis == "key"
    axis_code = lores.LORES_SCALE_KEY if key else lores.LORES_SCALE_VALUE
    step_bytes = sum(w.B * head_prec.count(c) * unit_bytes(c, w.dk, w.dv, in_bytes, w.per_channel,
                                                           key, win)
                     for c in range(6))
    st = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, head_prec, device=dev, scale_axis=axis_code,
                                 window=win)
    o = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)

    def step(t):
        i = (t - 1) % T_in
        lores.lores_decode_step(st, inputs["q"][i], inputs["k"][i], inputs["v"][i],
                                inputs["alpha"][i], inputs["beta"][i], w.delta, args.seed, t, o=o)

    n_launches_per_step = lores.lores_step_launches(st)

    def reset_state():
        nonlocal st
        st = lores.lores_state_alloc(w.B, w.H, w.dk, w.dv, head_prec, buf=st.buf,
                                     scale_axis=axis_code, window=win)

    print(f"[bench] warmup {W} eager steps", file=sys.stderr, flush=True)
    for t in range(1, W + 1):
        step(t)
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # timed region: K steps captured once as a HIP graph (one kernel node per
    # precision class and step), replayed after a warm replay from a fresh state
    mode = args.launch
    if mode == "graph":
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for t in range(1, K + 1):
                    step(t)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
        except Exception as exc:            # graphs unavailable: time eager launches
            print(f"[bench] graph capture failed ({exc}); timing eager launches",
                  file=sys.stderr, flush=True)
            mode = "eager"
    reset_state()
    print(f"[bench] timing {K} steps ({mode})", file=sys.stderr, flush=True)
    if mode == "graph":
        ms_total = timed(graph.replay)
    else:
        ms_total = timed(lambda: [step(t) for t in range(1, K + 1)])
    ms_step = ms_total / K
    ms_eager = timed(lambda: [step(t) for t in range(1, min(K, 256) + 1)]) / min(K, 256)

    # every launch of the timed region is a step kernel on torch's current
    # stream, which the events above bracket: the average launch duration is
    # the region's time over its launches
    avg_launch_ms = ms_total / (K * n_launches_per_step)
    print(f"[bench] {ms_step * 1e3:.2f} us/step ({mode}); {ms_eager * 1e3:.2f} us/step eager; "
          f"{n_launches_per_step} kernel launch(es) per step, {avg_launch_ms * 1e3:.2f} us per launch",
          file=sys.stderr, flush=True)

    achieved = step_bytes / n_launches_per_step / (avg_launch_ms * 1e-3) / 1e9
    profiled = not key and win == 1 and args.state == "assigned"
    traffic = load_traffic(w.key) if profiled else None
    valu_insts = load_valu(w.key) if profiled else None
    valu = None
    if valu_insts is not None:
        lane_ops = valu_insts * 64 / (avg_launch_ms * 1e-3)
        valu = {"achieved": lane_ops, "peak": VALU_PEAK_LANE_OPS,
                "unit": "VALU lane-instructions/s", "frac": lane_ops / VALU_PEAK_LANE_OPS,
                "insts_per_launch": valu_insts}

    # after the timed region: the same K steps repeated from a fresh state,
    # for the spread of the measurement (the reported value is the timed
    # region's alone)
    reps = []
    for _ in range(args.repeats):
        reset_state()
        reps.append(timed(graph.replay if mode == "graph" else
                          (lambda: [step(t) for t in range(1, K + 1)])) / K)
    reps.sort()
    result = {
        "metric": METRIC,
        "value": w.B * w.H * K / (ms_total * 1e-3),
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.key} {w.name}",
            "B": w.B, "H": w.H, "d_k": w.dk, "d_v": w.dv, "delta": w.delta,
            "decay": w.decay, "inputs": "bf16" if w.in_bf16 else "fp32",
            "state": {name: head_prec.count(c) for c, name in
                      enumerate(["fp32", "bf16", "int8", "int4", "int6", "fp8"]) if head_prec.count(c)},
            "rounding": "stochastic", "scale_axis": args.scale_axis, "window": win,
            "state_override": args.state,
            "parallelism": "single GPU",
        },
        "hbm_GBps_timed_loop": step_bytes / (ms_step * 1e-3) / 1e9,
        "launch": mode,
        "ms_per_step_eager": ms_eager,
        "us_per_launch": avg_launch_ms * 1e3,
        "algorithmic_bytes_per_step": step_bytes,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "kernel": "lores_step_kernel (fused dequant-update-readout-requant)",
            "launches_per_step": n_launches_per_step,
            "valu": valu,
            "limiter": limiter(achieved / HBM_PEAK_GBPS, valu["frac"] if valu else None),
        },
        "kernel_source_hash": kernel_source_hash(),
        "effective_bits": effective_bits(head_prec, w.dk, w.dv, key),
        "copy_reference": copy_reference(torch, step_bytes),
        "repeats": {"n": len(reps), "ms_per_step_median": reps[len(reps) // 2] if reps else None,
                    "ms_per_step_min": reps[0] if reps else None,
                    "ms_per_step_max": reps[-1] if reps else None},
    }
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inputs, head_prec, args.cpu_seconds, args.seed,
                                              args.scale_axis, win, args.cpu_workers)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
