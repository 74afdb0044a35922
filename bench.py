#!/usr/bin/env python3
"""Benchmark of the routed expert group (the hot path) on one MI355X.

A step is one dqg_expert_group call: stage x, stream every needed weight
byte of the token batch's routed experts and the shared expert, decode,
dot, SwiGLU, down projection and the rank-order weighted combine, y written.
The default workload is the int4-g32 group: 256 resident experts of
H = 6144, I = 2048 plus a shared expert, top-8 routing, 1 token.

Inputs are resident in HBM before timing.  Every step takes a fresh
routing (ids uniform without replacement, weights the softmax of N(0,1)
logits) and a fresh x from a seeded pool, and the shared expert rotates
over several copies, so the 256 MB Infinity Cache cannot serve a step's
weights from the previous steps.

Prints one JSON line: the metric is weight-stream GB/s (algorithmic bytes:
codes + scales of each distinct expert the step needs, once, plus x and
y) over wall time; `roofline` is the whole call (one launch at one token,
two or three otherwise) timed with HIP events on its stream, its bytes
over the summed kernel time, with a per-launch breakdown in `launches`.
The steps run twice back to back: first with the wall clock only (value,
ms_per_step), then with events on every launch (roofline;
ms_per_step_with_events), because the events themselves add several us a
call to the wall clock;
`cpu_baseline` is the CPU oracle on a bounded sample of the same steps.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quant GEMV weight-stream GB/s (% of HBM peak); µs per top-8 expert MLP"
HBM_PEAK_GBS = 8000.0


def launch_stats(launches):
    """{kernel: (count, total ms, median, p10, p90 in us)} from [(kernel, ms)]."""
    import numpy as np
    by = {}
    for name, ms in launches:
        by.setdefault(name, []).append(ms)
    out = {}
    for name, v in by.items():
        a = np.asarray(v) * 1e3
        out[name] = (len(v), float(np.sum(v)), round(float(np.median(a)), 2), round(float(np.percentile(a, 10)), 2),
                     round(float(np.percentile(a, 90)), 2))
    return out


def gpu_clocks():
    """The GPU's current clock levels as rocm-smi reports them (a child process), or None.

    None under a profiler that preloads itself into child processes: rocm-smi
    starts through an interpreter hop, an exec the preloaded child may not do."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        d = json.loads(r.stdout)
        card = next(iter(d.values()))
        return {k: v for k, v in card.items() if "clock" in k.lower()}
    except Exception:   # the clock state is context; its absence is not an error
        return None


def oracle_one_core(run_once, seconds, prepare=None):
    """(calls, seconds) of run_once(j) on one host thread, restoring the thread
    count; prepare(j), if given, runs before each call outside the clock."""
    import oracle
    n = oracle.get_threads()
    oracle.set_threads(1)
    try:
        spent, calls = 0.0, 0
        while spent < seconds:
            if prepare:
                prepare(calls)
            t = time.perf_counter()
            run_once(calls)
            spent += time.perf_counter() - t
            calls += 1
        return calls, spent
    finally:
        oracle.set_threads(n)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def host_cpu() -> dict:
    """The host's CPU model (/proc/cpuinfo), its logical CPU count (nproc)
    and the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_usable": usable}


KERNEL_SOURCES = ["dequant_gemv_expert_amd/csrc/dqg_kernels.hip", "dequant_gemv_expert_amd/csrc/dqg_api.cpp",
                  "dequant_gemv_expert_amd/csrc/dqg_internal.h"]
TRAFFIC_PROFILE = "profiles/group_int4g32_s1_traffic.md"


def kernel_sources_sha256() -> str:
    """SHA-256 of the kernel sources' code: comments and whitespace removed,
    so that only a change to the code itself voids a recorded profile."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)   # block comments
        src = re.sub(r"//[^\n]*", " ", src)                  # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def profiled_traffic(kernel: str):
    """HBM bytes per launch of `kernel` (or per call of "a+b", the sum over its
    launches) from the committed rocprofv3 counter summary, or None when the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic:"):
                key, _, val = line[len("traffic:"):].strip().partition("=")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    total = 0
    for name in kernel.split("+"):   # a call's launches, joined by "+": their sum
        v = fields.get(f"bytes_per_launch.{name}")
        if not v:
            return None
        total += int(float(v))
    return total


def matrix_bytes(m) -> int:
    n = m.q.nbytes + (0 if m.scales is None else m.scales.nbytes)
    if m.q2 is not None:
        n += m.q2.nbytes
    return n


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="int4g32_expert_group_256top8_shared")
    ap.add_argument("--tokens", type=int, default=None,
                    help="token batch (default: the workload's first; any S for the dense GEMV workloads)")
    ap.add_argument("--pool", type=int, default=1024, help="distinct routings drawn")
    ap.add_argument("--shared-copies", type=int, default=12)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gate-up", action="store_true",
                    help="dense workloads: time dqg_gate_up on two matrices of the workload's shape")
    ap.add_argument("--swiglu-limit", type=float, default=None,
                    help="clamp the experts' SwiGLU at this limit (expert-group workloads)")
    ap.add_argument("--activation", choices=("swiglu", "v4"), default="swiglu",
                    help="the experts' activation: the (clamped) SwiGLU, or DeepSeek V4's rounding form "
                         "(expert-group workloads)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only measure the plain streaming read (dqg_read_bytes): one pass over a 4.25 GiB "
                         "buffer, and reads the size of this library's launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch) 5 times, the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the path is measured "
              "on one GPU's share)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)
        return

    import synth
    import dequant_gemv_expert_amd as dq
    from dequant_gemv_expert_amd import _lib as L

    if args.stream_ceiling:
        return bench_stream(args)
    c = synth.WORKLOADS[args.workload]
    if c["kind"] == "gemv":
        return bench_gemv(args, c)
    if c["kind"] == "expert":
        return bench_expert(args, c)
    if c["kind"] != "group":
        raise SystemExit("bench.py times the expert-group, single-expert and dense GEMV workloads")
    S = args.tokens or c["S"][0]
    E, k, H, I, fmt, gs, seed = c["E"], c["k"], c["H"], c["I"], c["fmt"], c["gs"], c["seed"]
    n_shared = args.shared_copies if c["shared"] else 0
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)

    # -- resident experts ------------------------------------------------
    t0 = time.time()
    from concurrent.futures import ThreadPoolExecutor
    n_total = E + n_shared
    experts = [None] * n_total
    exp_bytes = gu_bytes = down_bytes = 0
    with ThreadPoolExecutor(16) as ex:
        for b0 in range(0, n_total, 16):
            idx = list(range(b0, min(n_total, b0 + 16)))
            hs = list(ex.map(lambda i: synth.expert(fmt, H, I, gs, seed, i), idx))
            for i, h in zip(idx, hs):
                experts[i] = dq.Expert.upload(h)
                if i == 0:
                    gu_bytes = matrix_bytes(h.gate) + matrix_bytes(h.up)
                    down_bytes = matrix_bytes(h.down)
                    exp_bytes = gu_bytes + down_bytes
    table = dq.ExpertTable(experts)
    if args.swiglu_limit is not None:
        table.set_swiglu_limit(args.swiglu_limit)
    if args.activation == "v4":
        table.set_activation(dq.DQG_ACT_SWIGLU_V4)
    torch.cuda.synchronize()
    log(f"[bench] {dev_name}: {n_total} experts resident ({n_total * exp_bytes / 1e9:.2f} GB) "
        f"in {time.time() - t0:.1f}s")

    # -- routing and activation pool ---------------------------------------
    P = args.pool
    ids = np.empty((P, S, k), np.int32)
    w = np.empty((P, S, k), np.float32)
    for p in range(P):
        ids[p], w[p] = synth.routing(S, E, k, seed, 7, S, p)
    x = synth.activations(P * S, H, seed, 8, S).reshape(P, S, H)
    union = np.array([len(np.unique(ids[p])) for p in range(P)])
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    x_d = torch.from_numpy(x).cuda()
    y_d = torch.empty((S, H), dtype=torch.float32, device="cuda")
    scratch = table.scratch(S, k)
    lib = L.load()
    stream = torch.cuda.current_stream().cuda_stream
    nbytes_scratch = scratch.numel()
    shared_of = (lambda i: E + i % n_shared) if n_shared else (lambda i: -1)
    n_sh = 1 if n_shared else 0

    def call_args(i):
        p = i % P
        return (table.handle, S, k, ids_d[p].data_ptr(), w_d[p].data_ptr(), shared_of(i),
                x_d[p].data_ptr(), y_d.data_ptr(), scratch.data_ptr(), nbytes_scratch, stream)

    plan = [call_args(i) for i in range(args.warmup + args.steps)]
    io_bytes = S * H * 4 * 2                       # x read, y written
    h_bytes = (S * k + S * n_sh) * I * 4           # h written by gate/up, read by down

    def step_bytes(i):
        units = union[i % P] + n_sh
        return units * exp_bytes + io_bytes

    def step_bytes_gate_up(i):
        return (union[i % P] + n_sh) * gu_bytes + S * H * 4 + h_bytes

    # -- warmup ------------------------------------------------------------
    fn = lib.dqg_expert_group
    for i in range(args.warmup):
        rc = fn(*plan[i])
        if rc:
            raise RuntimeError(dq.dqg_last_error())
    torch.cuda.synchronize()

    # -- timed region 1: the steps back to back, wall clock only ------------
    K = args.steps

    def run_steps():
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(args.warmup, args.warmup + K):
            rc = fn(*plan[i])
            if rc:
                raise RuntimeError(dq.dqg_last_error())
        torch.cuda.synchronize()
        return time.perf_counter() - t

    t_wall = run_steps()
    # -- timed region 2: the same steps with HIP events around every launch,
    #    on the launch's stream (the events add about 8 us a call to the wall
    #    clock, which is why value comes from region 1) ---------------------
    clocks = gpu_clocks()
    dq.dqg_prof_begin(3 * K)   # at most three launches a call (DeepSeek V4's activation)
    t_wall_events = run_steps()
    launches = dq.dqg_prof_end_launches(3 * K)
    pstats = launch_stats(launches)
    prof = {name: v[:2] for name, v in pstats.items()}
    per_call = len(launches) // K
    if per_call * K != len(launches) or per_call not in (1, 2, 3):
        raise RuntimeError(f"{len(launches)} launches timed for {K} calls")
    # kernel time of each call: the sum of its launches' durations
    call_us = [sum(ms for _, ms in launches[j * per_call:(j + 1) * per_call]) * 1e3 for j in range(K)]

    total_bytes = sum(step_bytes(i) for i in range(args.warmup, args.warmup + K))
    timed = range(args.warmup, args.warmup + K)   # region 2 times every call's launches
    ms_per_step = t_wall * 1e3 / K
    value = total_bytes / t_wall / 1e9
    kernel_ms = sum(call_us) * 1e-3
    achieved = total_bytes / (kernel_ms * 1e-3) / 1e9
    kernels = [name for name, _ in launches[:per_call]]
    group_kernel = "+".join(kernels)
    # per-launch breakdown: the gate/up launch moves its weights, x and h; down its weights, h and y
    breakdown = {}
    for name in kernels:
        n_k, ms_k = prof[name]
        if name == "group_gate_up":
            b = sum(step_bytes_gate_up(i) for i in timed)
        elif name == "group_down":
            b = sum((union[i % P] + n_sh) * down_bytes + h_bytes + S * H * 4 for i in timed)
        elif name == "group_fused":
            b = total_bytes
        else:
            b = None
        breakdown[name] = {"avg_us": round(ms_k / n_k * 1e3, 2), "median_us": pstats[name][2],
                           "p10_us": pstats[name][3], "p90_us": pstats[name][4],
                           "traffic": profiled_traffic(name) if (S == 1 and args.workload ==
                                      "int4g32_expert_group_256top8_shared") else None,
                           **({"bytes_per_launch": round(b / n_k), "achieved": round(b / (ms_k * 1e-3) / 1e9, 1)}
                              if b else {})}
    pc = np.asarray(call_us)
    log(f"[bench] {K} steps: {ms_per_step * 1e3:.1f} us/step wall, {value:.0f} GB/s; kernel time "
        f"{np.mean(pc):.1f} us a call ({achieved:.0f} GB/s, {achieved / HBM_PEAK_GBS:.3f} of peak) over "
        + ", ".join(f"{k} {v['avg_us']} us" for k, v in breakdown.items())
        + f"; mean union {union.mean():.2f} experts + {n_sh} shared")

    # -- CPU oracle on a bounded sample -------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cache = {}

        def host_expert(e):
            if e not in cache:
                cache[e] = synth.expert(fmt, H, I, gs, seed, e)
            return cache[e]

        class View:
            def __len__(self):
                return n_total

            def __getitem__(self, e):
                return host_expert(int(e))

        limit = math.inf if args.swiglu_limit is None else args.swiglu_limit

        def oracle_group(*a):
            if args.activation == "v4":
                return oracle.expert_group_v4(*a, limit)
            return oracle.expert_group(*a, limit)

        threads = oracle.get_threads()
        spent, calls, cbytes = 0.0, 0, 0
        while spent < args.cpu_seconds and calls < P:
            i = args.warmup + calls
            p = i % P
            for e in set(ids[p].ravel().tolist()) | ({shared_of(i)} if n_shared else set()):
                host_expert(e)   # drawn before the clock starts
            t = time.perf_counter()
            oracle_group(View(), ids[p], w[p], shared_of(i), x[p])
            spent += time.perf_counter() - t
            calls += 1
            cbytes += step_bytes(i)
            if len(cache) > 64:
                cache.clear()
        cpu = {"value": round(cbytes / spent / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{calls} expert-group calls ({S} token(s), top-{k} of {E}"
                         f"{' + shared' if n_sh else ''}) from the same routing pool, {spent:.1f} s",
               "us_per_call": round(spent / calls * 1e6, 1), **host_cpu()}

        def draw(j):   # the call's experts, drawn before the clock starts
            i = args.warmup + (j % calls)
            if len(cache) > 64:
                cache.clear()
            for e in set(ids[i % P].ravel().tolist()) | ({shared_of(i)} if n_shared else set()):
                host_expert(e)

        def one_call(j):   # the same calls again, on one host thread
            i = args.warmup + (j % calls)
            oracle_group(View(), ids[i % P], w[i % P], shared_of(i), x[i % P])

        c1, s1 = oracle_one_core(one_call, max(1.0, args.cpu_seconds / 3), draw)
        cpu["value_1core"] = round(sum(step_bytes(args.warmup + (j % calls)) for j in range(c1)) / s1 / 1e9, 3)
        log(f"[bench] cpu oracle: {cpu['value']} GB/s on {threads} threads ({calls} calls), "
            f"{cpu['value_1core']} GB/s on 1")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "ms_per_step_with_events": round(t_wall_events * 1e3 / K, 5),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": S, "top_k": k, "experts": E,
                   "shared_expert": bool(n_sh), "H": H, "I": I, "format": f"fmt {fmt}, gs {gs}",
                   "routing_pool": P, "shared_copies": n_shared, "device": dev_name,
                   **({} if args.swiglu_limit is None else {"swiglu_limit": args.swiglu_limit}),
                   **({} if args.activation == "swiglu" else {"activation": "deepseek_v4_rounding"})},
        "roofline": {"kernel": group_kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(group_kernel) if (S == 1 and args.workload ==
                                "int4g32_expert_group_256top8_shared") else None,
                     "scope": "the whole call: every launch of it, algorithmic bytes over summed kernel time",
                     "avg_us": round(float(np.mean(pc)), 2), "median_us": round(float(np.median(pc)), 2),
                     "p10_us": round(float(np.percentile(pc, 10)), 2), "p90_us": round(float(np.percentile(pc, 90)), 2),
                     "bytes_per_call": round(total_bytes / K), "timed_calls": K, "launches_per_call": per_call},
        "roofline_group": {"kernel_time_frac": round(achieved / HBM_PEAK_GBS, 4),
                           "wall_frac": round(value / HBM_PEAK_GBS, 4),
                           "kernel_us_per_call": round(float(np.mean(pc)), 2),
                           "wall_us_per_call": round(ms_per_step * 1e3, 2)},
        "launches": breakdown,
        "gpu_clocks": clocks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    table.close()


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense f16 matrix-core peak


def bench_gemv(args, c):
    """A dense quantised matrix (dqg_matmul) at --tokens S: one step is one call.

    Distinct device copies of the matrix (about 2 GB in all) rotate so that
    the Infinity Cache cannot serve a step's weights.  The library picks the
    route: the per-row route streams the weights (HBM-bound, GB/s); the
    matrix-core GEMM (from a format's cut-over on) is reported in TFLOP/s of
    useful products against the f16 peak.  The route is read off the timed
    launches.  With --gate-up a step is one dqg_gate_up call on a gate and an
    up matrix of the workload's shape.
    """
    import numpy as np
    import torch
    import synth
    import dequant_gemv_expert_amd as dq

    S = args.tokens or c["S"][0]
    fmt, O, K, gs, seed = c["fmt"], c["O"], c["K"], c["gs"], c["seed"]
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)
    gu = args.gate_up
    hm = synth.matrix(fmt, O, K, gs, seed, 0)
    hu = synth.matrix(fmt, O, K, gs, seed, 1) if gu else None
    w_bytes = matrix_bytes(hm) * (2 if gu else 1)
    copies = max(2, min(256, (2 << 30) // w_bytes))
    mats = [(dq.Matrix.upload(hm), dq.Matrix.upload(hu) if gu else None) for _ in range(copies)]
    x = torch.from_numpy(synth.activations(S, K, seed, 9, S)).cuda()
    y = torch.empty((S, O), dtype=torch.float32, device="cuda")
    log(f"[bench] {dev_name}: {copies} copies of {args.workload}{' (gate and up)' if gu else ''} "
        f"({w_bytes / 1e6:.2f} MB each), S = {S}")
    # ctypes arguments prepared up front, so the timed loop is the C calls
    import ctypes
    from dequant_gemv_expert_amd import _lib as L
    stream = torch.cuda.current_stream().cuda_stream
    if gu:
        fn = L.load().dqg_gate_up
        plan = [(ctypes.byref(g.struct), ctypes.byref(u.struct), x.data_ptr(), S, y.data_ptr(), stream)
                for g, u in mats]
    else:
        fn = L.load().dqg_matmul
        plan = [(ctypes.byref(g.struct), x.data_ptr(), S, y.data_ptr(), stream) for g, _ in mats]

    def call(i):
        rc = fn(*plan[i % copies])
        if rc:
            raise RuntimeError(dq.dqg_last_error())

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    K_steps = args.steps

    def run_steps():
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(K_steps):
            call(args.warmup + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t

    t_wall = run_steps()                     # region 1: wall clock only
    clocks = gpu_clocks()
    dq.dqg_prof_begin(2 * K_steps)           # region 2: events on every launch (split-K: two a call)
    t_wall_events = run_steps()
    launches = dq.dqg_prof_end_launches(2 * K_steps)
    prof = {name: v[:2] for name, v in launch_stats(launches).items()}
    # kernel time per call: a call's launch, plus its split-K reduce when it has one
    call_us = []
    for name, ms in launches:
        if name == "gemm_reduce" and call_us:
            call_us[-1] += ms * 1e3
        else:
            call_us.append(ms * 1e3)
    pc = np.asarray(call_us)
    pct = {"median_us": round(float(np.median(pc)), 2), "p10_us": round(float(np.percentile(pc, 10)), 2),
           "p90_us": round(float(np.percentile(pc, 90)), 2)}
    # the route the library took (the kernel whose launches were timed)
    routes = ("gemm_gate_up", "gate_up") if gu else ("gemm", "matmul")
    kname = max(routes, key=lambda k: prof.get(k, (0, 0.0))[0])
    gemm = kname == routes[0]
    n_k, ms_k = prof.get(kname, (0, 0.0))
    if gemm and prof.get("gemm_reduce", (0, 0.0))[0]:   # split-K: the partials' sum is part of the call
        ms_k += prof["gemm_reduce"][1]
        kname += "+gemm_reduce"
    avg_s = ms_k * 1e-3 / max(n_k, 1)
    step_bytes = w_bytes + S * K * 4 + S * O * 4
    flops = 2.0 * S * O * K * (2 if gu else 1)
    value = step_bytes * K_steps / t_wall / 1e9
    if gemm:
        achieved = flops / avg_s / 1e12 if avg_s > 0 else None
        roof = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 2) if achieved else None,
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4) if achieved else None, "traffic": None,
                "avg_us": round(avg_s * 1e6, 2), "flops_per_launch": flops, "timed_launches": n_k, **pct}
    else:
        achieved = step_bytes / avg_s / 1e9 if avg_s > 0 else None
        roof = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                "traffic": None, "avg_us": round(avg_s * 1e6, 2), "bytes_per_launch": step_bytes,
                "timed_launches": n_k, **pct}
    log(f"[bench] {K_steps} steps: {t_wall / K_steps * 1e6:.1f} us/step wall; {kname} kernel "
        f"{avg_s * 1e6:.1f} us avg; {flops / avg_s / 1e12 if avg_s else 0:.1f} TFLOP/s, "
        f"{step_bytes / avg_s / 1e9 if avg_s else 0:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        rows = max(1, min(O, int(O * 0.05)))
        srows = -(-rows // synth.FP8_BLOCK) if fmt == synth.FMT_FP8_BLOCK else rows   # whole scale blocks

        def head(m):   # the first rows of a matrix
            return synth.QMatrix(m.fmt, rows, m.K, m.gs, m.q[:rows], None if m.q2 is None else m.q2[:rows],
                                 None if m.scales is None else m.scales[:srows])
        sub = head(hm)
        subu = head(hu) if gu else None
        xs = x.cpu().numpy()
        spent, calls = 0.0, 0
        while spent < args.cpu_seconds and calls < 1_000_000:
            t = time.perf_counter()
            if gu:
                oracle.gate_up(sub, subu, xs)
            else:
                oracle.gemv(sub, xs)
            spent += time.perf_counter() - t
            calls += 1
        per_call = spent / calls * O / rows   # the whole matrix, scaled from the row sample

        def rate(t_call):
            return round((step_bytes / t_call / 1e9) if not gemm else (flops / t_call / 1e12), 4)

        cpu = {"value": rate(per_call),
               "unit": "GB/s" if not gemm else "TFLOP/s", "cores": oracle.get_threads(), "kind": "oracle",
               "sample": f"{calls} oracle {'gate_up calls' if gu else 'GEMVs'} of the first {rows} of {O} rows "
                         f"at S = {S}, {spent:.1f} s, scaled to the whole matrix", **host_cpu()}

        def one_call(j):   # the same sample on one host thread
            if gu:
                oracle.gate_up(sub, subu, xs)
            else:
                oracle.gemv(sub, xs)

        c1, s1 = oracle_one_core(one_call, max(1.0, args.cpu_seconds / 3))
        cpu["value_1core"] = rate(s1 / c1 * O / rows)
        log(f"[bench] cpu oracle: {cpu['value']} {cpu['unit']} on {cpu['cores']} threads, {cpu['value_1core']} on 1")

    out = {
        "metric": (METRIC if not gemm else "quant GEMM TFLOP/s (prefill, useful products)")
                  + (" [gate_up]" if gu else ""),
        "value": round(value, 2) if not gemm else round(flops * K_steps / t_wall / 1e12, 3),
        "unit": "GB/s" if not gemm else "TFLOP/s",
        "n_gpus": 1, "steps": K_steps, "warmup": args.warmup,
        "ms_per_step": round(t_wall / K_steps * 1e3, 5), "us_per_call": round(t_wall / K_steps * 1e6, 2),
        "ms_per_step_with_events": round(t_wall_events / K_steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload + (" gate_up" if gu else ""), "tokens": S, "O": O, "K": K,
                   "format": f"fmt {fmt}, gs {gs}",
                   "copies": copies, "route": "gemm" if gemm else "gemv", "device": dev_name},
        "roofline": roof,
        "gpu_clocks": clocks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_stream(args):
    """The plain streaming read (dqg_read_bytes) on one MI355X.

    One pass over a 4.25 GiB buffer per launch (the long-stream ceiling),
    then reads of the byte counts of this library's launches (the dense
    int4-g32 6144 x 6144 matrix, the int4-g32 group's down launch, gate/up
    launch and whole call at one token, and the two launches of one int4-g32
    expert of H 6144, I 2048), each launch at its own
    offset so that the Infinity Cache cannot serve it.  HIP events on every
    launch give its duration.
    """
    import numpy as np
    import torch
    import dequant_gemv_expert_amd as dq

    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)
    total = 4352 << 20
    buf = torch.empty(total, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    sizes = {"whole_buffer": total, "gemv_int4g32_6144x6144": 23642112, "group_int4g32_down": 70778880,
             "group_int4g32_gate_up": 141557760, "group_int4g32_call": 212336640,
             "expert_int4g32_gate_up": 15728640, "expert_int4g32_down": 7864320}
    results = {}
    for name, n in sizes.items():
        n = n // 1024 * 1024
        launches = 10 if n == total else args.steps
        offsets = [0] if n == total else [(i * n) % (total - n) // 4096 * 4096 for i in range(launches + args.warmup)]
        for i in range(args.warmup if n != total else 2):
            dq.dqg_read_bytes(buf, sink, n, offsets[i % len(offsets)])
        torch.cuda.synchronize()
        dq.dqg_prof_begin(launches)
        for i in range(launches):
            dq.dqg_read_bytes(buf, sink, n, offsets[(i + args.warmup) % len(offsets)] if n != total else 0)
        torch.cuda.synchronize()
        ms = [m for _, m in dq.dqg_prof_end_launches(launches)]
        avg = float(np.mean(ms)) * 1e-3
        results[name] = {"bytes": n, "launches": len(ms), "avg_us": round(avg * 1e6, 2),
                         "median_us": round(float(np.median(ms)) * 1e3, 2), "GB/s": round(n / avg / 1e9, 1),
                         "frac": round(n / avg / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] read {n / 1e6:.1f} MB: {avg * 1e6:.2f} us a launch, {n / avg / 1e9:.0f} GB/s")
    whole = results["whole_buffer"]
    out = {"metric": "plain streaming read GB/s (the weight streams' ceiling)", "value": whole["GB/s"],
           "unit": "GB/s", "n_gpus": 1, "steps": whole["launches"], "warmup": 2, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": "stream_read", "bytes": total, "device": dev_name},
           "roofline": {"kernel": "read", "bound": "hbm", "achieved": whole["GB/s"], "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": whole["frac"], "traffic": None, "avg_us": whole["avg_us"]},
           "by_size": results, "gpu_clocks": gpu_clocks(), "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def bench_expert(args, c):
    """One expert MLP at one token: dqg_expert_group with a single routed
    expert of weight 1 and no shared expert, so y = down(SwiGLU(gate x, up x)).

    Distinct device copies of the expert (about 2 GB in all) rotate so that
    the Infinity Cache cannot serve a step's weights.  Reported in us per
    call and as weight-stream GB/s over the summed kernel time of the call's
    two launches.
    """
    import numpy as np
    import torch
    import synth
    import dequant_gemv_expert_amd as dq
    from dequant_gemv_expert_amd import _lib as L

    S, k = 1, 1
    fmt, H, I, gs, seed = c["fmt"], c["H"], c["I"], c["gs"], c["seed"]
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)
    he = synth.expert(fmt, H, I, gs, seed, 0)
    exp_bytes = matrix_bytes(he.gate) + matrix_bytes(he.up) + matrix_bytes(he.down)
    copies = max(2, min(256, (2 << 30) // exp_bytes))
    de = dq.Expert.upload(he)
    table = dq.ExpertTable([de] + [dq.Expert.upload(he) for _ in range(copies - 1)])
    x = synth.activations(S, H, seed, 9)
    x_d = torch.from_numpy(x).cuda()
    y_d = torch.empty((S, H), dtype=torch.float32, device="cuda")
    ids = torch.arange(copies, dtype=torch.int32, device="cuda").reshape(copies, 1, 1)
    w = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    scratch = table.scratch(S, k)
    lib = L.load()
    stream = torch.cuda.current_stream().cuda_stream
    plan = [(table.handle, S, k, ids[i].data_ptr(), w.data_ptr(), -1, x_d.data_ptr(), y_d.data_ptr(),
             scratch.data_ptr(), scratch.numel(), stream) for i in range(copies)]
    log(f"[bench] {dev_name}: {copies} copies of {args.workload} ({exp_bytes / 1e6:.2f} MB each)")

    def call(i):
        rc = lib.dqg_expert_group(*plan[i % copies])
        if rc:
            raise RuntimeError(dq.dqg_last_error())

    for i in range(args.warmup):
        call(i)
    K = args.steps

    def run_steps():
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(K):
            call(args.warmup + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t

    t_wall = run_steps()
    clocks = gpu_clocks()
    dq.dqg_prof_begin(2 * K)
    t_wall_events = run_steps()
    launches = dq.dqg_prof_end_launches(2 * K)
    per_call = len(launches) // K
    if per_call * K != len(launches):
        raise RuntimeError(f"{len(launches)} launches timed for {K} calls")
    call_us = np.asarray([sum(ms for _, ms in launches[j * per_call:(j + 1) * per_call]) * 1e3 for j in range(K)])
    pstats = launch_stats(launches)
    step_bytes = exp_bytes + S * H * 4 * 2 + 2 * S * I * 4   # weights, x and y, h written and read
    kernel_s = float(np.mean(call_us)) * 1e-6
    achieved = step_bytes / kernel_s / 1e9
    value = step_bytes * K / t_wall / 1e9
    breakdown = {name: {"avg_us": round(v[1] / v[0] * 1e3, 2), "median_us": v[2], "p10_us": v[3], "p90_us": v[4]}
                 for name, v in pstats.items()}
    log(f"[bench] {K} steps: {t_wall / K * 1e6:.1f} us/step wall; kernel time {kernel_s * 1e6:.1f} us a call "
        f"({achieved:.0f} GB/s, {achieved / HBM_PEAK_GBS:.3f} of peak) over "
        + ", ".join(f"{n} {v['avg_us']} us" for n, v in breakdown.items()))

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        spent, calls = 0.0, 0
        while spent < args.cpu_seconds and calls < 100000:
            t = time.perf_counter()
            oracle.expert_group([he], np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), None, x)
            spent += time.perf_counter() - t
            calls += 1
        cpu = {"value": round(step_bytes * calls / spent / 1e9, 3), "unit": "GB/s", "cores": oracle.get_threads(),
               "kind": "oracle", "sample": f"{calls} oracle expert MLP calls (1 token), {spent:.1f} s",
               "us_per_call": round(spent / calls * 1e6, 1), **host_cpu()}

        def one_call(j):
            oracle.expert_group([he], np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), None, x)

        c1, s1 = oracle_one_core(one_call, max(1.0, args.cpu_seconds / 3))
        cpu["value_1core"] = round(step_bytes * c1 / s1 / 1e9, 3)
        log(f"[bench] cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads, {cpu['value_1core']} on 1")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(t_wall / K * 1e3, 5), "us_per_call": round(t_wall / K * 1e6, 2),
        "ms_per_step_with_events": round(t_wall_events / K * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": S, "H": H, "I": I, "format": f"fmt {fmt}, gs {gs}",
                   "copies": copies, "device": dev_name},
        "roofline": {"kernel": "+".join(n for n, _ in launches[:per_call]), "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "scope": "the whole call: both launches, algorithmic bytes over summed kernel time",
                     "avg_us": round(kernel_s * 1e6, 2), "median_us": round(float(np.median(call_us)), 2),
                     "bytes_per_call": step_bytes, "timed_calls": K, "launches_per_call": per_call},
        "launches": breakdown, "gpu_clocks": clocks, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    table.close()


if __name__ == "__main__":
    main()
