"""Benchmark of the MoE dispatch/combine core on one MI355X.

One step = the whole path over one synthetic batch already resident in HBM:
moe_route_dispatch_layout (routing and layout; one launch for batches of at
most 4096 assignments) -> moe_dispatch_permute -> moe_combine_reduce (the
expert is the identity: combine reads the send buffer). The same step with
moe_route_topk and moe_dispatch_layout as separate calls is timed beside it
("four_call_step_us"). W untimed warm-up steps, then exactly K timed steps between
device synchronisations with HIP events only at the two ends (an event
between calls leaves the GPU idle for a few microseconds). The steps are
eager launches, each call's device pointers bound once before timing (as a
C caller holds them); --graph times replays of a HIP graph that holds the
four launches instead. A second pass of K steps records an event pair
around every call, on the stream the kernels run on, for the per-call
durations and the roofline of the dominant kernel.

Prints ONE JSON line on stdout. `value` is algorithmic HBM bytes per step /
step time (GB/s) on the largest workload (--workload, fine_grained by
default); tokens/s and the fraction of the 8 TB/s peak ride along.
Algorithmic bytes count every array each call must read once and write once,
for kept rows only:
  route    read T*E*4 (+E*4 bias)              write 2*T*k*4
  layout   read T*k*4                          write T*k*4 + N*4 + (3E + 2R + 2)*4
  permute  read T*k*4 + T_read*H*2             write N*H*2
  combine  read 2*T*k*4 + N*H*2 + T*H*2*(residual + shared)   write T*H*2
with N kept rows and T_read tokens that have at least one kept replica (both
read from the path's own outputs after the timed region).

The other workloads (--also, by default the two other prefill workloads and
the decode and tiny ones) are measured the same way and reported under
"workloads": step time, GB/s, share of peak, tokens/s, per-call times, the
dominant kernel's roofline and the synthetic floor for their byte mix.

The synthetic floor is moe_hbm_floor: a hand-written contiguous streaming
kernel that reads and writes given byte counts with the row kernels' 16-byte
lane accesses and nothing else. It is timed like the step at the step's own
read and write volumes, and at each of the permute's and the combine's, plus
a write-only stream of the permute's write bytes (the write ceiling), each
with non-temporal and with ordinary stores, keeping the faster. The gap
between a call and its floor is overhead the path owns. On dropless
workloads the permute and the combine are also timed with every token's
replicas at rows t*k .. t*k + k - 1 ("token_order_rows_us"), which
separates the cost of the layout's scattered rows from the kernels' own.

After the path, further measurements are reported under "next_rows", none
part of `value`:
  * the same step with the FP8 dispatch payload (moe_dispatch_permute_fp8 in
    place of the bf16 permute), on this workload and on each prefill workload
    under --also;
  * the receive-side regroup on the same buffers (the send buffer read as R
    source segments);
  * the tile-signalled return: a stand-in expert GEMM on those segments whose
    tiles are returned as they finish, against the GEMM then a copy, on this
    workload and on each prefill workload under --also.

Alongside: the spread of single-step times (a third pass with one event
between steps); the same spread from a cold cache (a fourth pass, each step
after a 1 GiB scratch read that evicts the Infinity Cache); a fifth pass
with two batches in flight on two streams, each with its own outputs, whose
results must equal a step on its own bit for bit ("pipelined_two_streams");
and the load imbalance read from the layout's own counts ("load").

The CPU-baseline leg times the plain C oracle on the same host arrays:
whole passes on one core for about --cpu-seconds, median pass.

Two offline modes read rocprofv3 output written by earlier runs of this
script and exit: --summarize DIR prints a markdown table of a
`--kernel-trace --stats` run, and --write-traffic FETCH_DIR WRITE_DIR turns
two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs into the per-kernel traffic
records under profiles/ (scaled by the floor kernel's own counts).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "combine_kernel": "combine_route_topk_amd/csrc/combine.hip",
    "permute_kernel": "combine_route_topk_amd/csrc/permute.hip",
    "permute_fp8_kernel": "combine_route_topk_amd/csrc/fp8.hip",
    "regroup_rows_kernel": "combine_route_topk_amd/csrc/regroup.hip",
}
PREFILL = ("prefill_capacity", "ragged_dropless", "fine_grained")
CONSUMER_COUNTS = (16, 24, 32, 0)   # dedicated consumer blocks tried by the tile-signalled return
FLOOR_CALIBRATION_BYTES = 1 << 30   # the floor kernel run as a copy of this size, for counter scaling


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="fine_grained",
                   help="the workload `value` is measured on: one of "
                        + ", ".join(w.name for w in synthetic.WORKLOADS.values()))
    p.add_argument("--also", default="prefill_capacity,ragged_dropless,decode,tiny",
                   help="comma-separated further workloads reported under `workloads` ('' for none)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time replays of a captured HIP graph of the step instead of eager launches")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cold-cache pass (each step after a 1 GiB scratch read)")
    p.add_argument("--no-floor", action="store_true", help="skip the synthetic floor")
    p.add_argument("--no-token-order", action="store_true",
                   help="skip the permute and combine timed with every token's rows in token order")
    p.add_argument("--no-pipelined", action="store_true",
                   help="skip the pass with two batches in flight on two streams")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8-payload step (next_rows)")
    p.add_argument("--no-tile-return", action="store_true",
                   help="skip the tile-signalled return (next_rows); its cooperative launch is also "
                        "left out of any run under a profiler")
    p.add_argument("--no-regroup", action="store_true", help="skip the receive-side regroup (next_rows)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="rough CPU time budget of the oracle baseline")
    p.add_argument("--route-groups", default=None, metavar="G,M",
                   help="route with moe_route_topk_grouped: at most M of G expert groups per token")
    p.add_argument("--calibrate", action="store_true",
                   help="also run the floor kernel as a 1 GiB copy (the counter calibration launch)")
    p.add_argument("--summarize", metavar="DIR", default=None,
                   help="print a markdown summary of a rocprofv3 --kernel-trace --stats output and exit")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                   help="write profiles/traffic_<kernel>_<workload>.json from two counter runs and exit")
    return p.parse_args(argv)


def workload_by_name(name):
    for i, w in synthetic.WORKLOADS.items():
        if name in (w.name, str(i)):
            return w
    raise SystemExit(f"unknown workload {name}")


def rw_bytes(w, N, T_read, has_bias):
    """Algorithmic (read, write) bytes of each call of one step."""
    T, H, E, k, R = w.T, w.H, w.E, w.k, w.R
    dense = (1 if w.residual else 0) + (1 if w.shared else 0)   # residual + shared
    return {
        "route": (T * E * 4 + (E * 4 if has_bias else 0), 2 * T * k * 4),
        "layout": (T * k * 4, T * k * 4 + N * 4 + (3 * E + 2 * R + 2) * 4),
        "permute": (T * k * 4 + T_read * H * 2, N * H * 2),
        "combine": (2 * T * k * 4 + N * H * 2 + T * H * 2 * dense, T * H * 2),
    }


def call_bytes(nbytes, name):
    """Algorithmic bytes of one call (route_layout: the two calls' bytes)."""
    return nbytes["route"] + nbytes["layout"] if name == "route_layout" else nbytes[name]


def algorithmic_bytes(w, N, T_read, has_bias):
    return {n: r + wr for n, (r, wr) in rw_bytes(w, N, T_read, has_bias).items()}


def source_hash(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or taken on a different version of the kernel's source."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def load_balance(demand, kept, dest_rows):
    """Load imbalance from the layout's own counts: max / mean per expert
    (demand and kept rows) and per destination, since a skewed router makes
    the busiest expert and the busiest destination set the time."""
    ratio = lambda a: round(float(a.max() / a.mean()), 3) if a.size and a.mean() > 0 else None
    return {"expert_demand_max_over_mean": ratio(demand), "expert_kept_max_over_mean": ratio(kept),
            "dest_rows_max_over_mean": ratio(dest_rows), "hot_dest_rows": int(dest_rows.max()),
            "dropped": int(demand.sum() - kept.sum())}


def host_cpu():
    """CPU model name (from /proc/cpuinfo) and the cores this process may run on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(w, d, budget_s):
    """Time the single-threaded C oracle over the same workload: whole passes
    (route, layout, permute, combine) until about budget_s seconds are spent,
    at least three; returns the median pass time and the pass count."""
    import oracle
    reps, times = 0, []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        idx, wt = oracle.route_topk(d["logits"], d["bias"], w.k)
        L = oracle.dispatch_layout(idx, w.E, w.R, w.capacity)
        N = int(L["expert_offsets"][-1])
        send = oracle.dispatch_permute(d["x"], L["pos"], max(N, 1))
        oracle.combine_reduce(send, L["pos"], wt, d["shared"], d["residual"])
        times.append(time.perf_counter() - t0)
        reps += 1
        del send
        # passes until the budget is spent (at least 3): the median of many
        if reps >= 3 and time.perf_counter() - t_start > budget_s:
            break
    return statistics.median(times), reps


# ---------------------------------------------------------------------------
# offline modes: rocprofv3 output -> summaries and traffic records
# ---------------------------------------------------------------------------

def _csv_rows(directory, suffix):
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short(name):
    """Kernel name without the namespace, argument list or launch suffix."""
    n = name.replace("moe::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    n = n.split("(")[0].replace("void ", "")
    return n.strip()


def summarize(directory):
    stats = _csv_rows(directory, "kernel_stats.csv")
    if not stats:
        raise SystemExit(f"no *kernel_stats.csv under {directory}")
    print("| kernel | calls | average us | min us | max us | total % |")
    print("|---|---|---|---|---|---|")
    # PyTorch's and the runtime's own kernels (input upload, bookkeeping) are left out
    ours = [r for r in stats if not r["Name"].startswith(("at::", "void at::", "__amd_rocclr"))]
    for r in sorted(ours, key=lambda r: -float(r["TotalDurationNs"])):
        print(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    # the floor kernel runs at several byte mixes, one pass after another
    # (the benchmark's order: step, permute, combine, write-only), each with
    # non-temporal then ordinary stores: split it into its passes, a pass
    # being a run of launches of one instance with one grid
    trace = sorted(_csv_rows(directory, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    passes = []
    for r in trace:
        name = _short(r["Kernel_Name"])
        if not name.startswith("floor_kernel"):
            continue
        key = (int(r["Grid_Size_X"]), name)
        if not passes or passes[-1][0] != key:
            passes.append((key, []))
        passes[-1][1].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if passes:
        names = ["step", "permute", "combine", "write-only"]
        print("\n| floor pass (benchmark order) | stores | grid (threads) | calls | average us |")
        print("|---|---|---|---|---|")
        for i, ((grid, name), v) in enumerate(passes):
            label = names[(i // 2) % 4] if len(passes) % 8 == 0 else str(i)
            kind = "non-temporal" if "<true>" in name else "ordinary"
            print(f"| {label} | {kind} | {grid} | {len(v)} | {sum(v) / len(v):.2f} |")


def _counter_means(directory, counter):
    """Mean per dispatch of `counter` (summed over its instances) by kernel name."""
    per_dispatch = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Dispatch_Id"], _short(r["Kernel_Name"]))
        per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    by_kernel = {}
    for (_, name), v in per_dispatch.items():
        by_kernel.setdefault(name, []).append(v)
    return {n: sum(v) / len(v) for n, v in by_kernel.items()}


def write_traffic(fetch_dir, write_dir, workload, commands):
    """Per-kernel HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled so that the floor kernel's calibration copy (1 GiB
    read, 1 GiB written) reads as exactly that many bytes."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    cal = [n for n in fetch if n.startswith("floor_kernel")]
    if len(cal) != 1:
        raise SystemExit("the counter runs need exactly one floor kernel, the calibration copy "
                         "(run the bench with --calibrate --no-floor)")
    fk = cal[0]
    gib_kib = FLOOR_CALIBRATION_BYTES / 1024
    fetch_scale, write_scale = gib_kib / fetch[fk], gib_kib / write[fk]
    out = []
    for kernel, rel in KERNEL_SOURCES.items():
        names = [n for n in fetch if n.startswith(kernel) and n in write]
        if not names:
            continue
        name = max(names, key=lambda n: fetch[n])
        nbytes = fetch[name] * 1024 * fetch_scale + write[name] * 1024 * write_scale
        rec = {"kernel": name, "workload": workload, "source": rel, "source_sha256_16": source_hash(rel),
               "fetch_size_kib_per_launch": round(fetch[name], 1),
               "write_size_kib_per_launch": round(write[name], 1),
               "calibration": {"kernel": fk, "bytes_read": FLOOR_CALIBRATION_BYTES,
                               "bytes_written": FLOOR_CALIBRATION_BYTES,
                               "fetch_size_kib": round(fetch[fk], 1), "write_size_kib": round(write[fk], 1)},
               "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
               "hbm_bytes_per_launch": int(round(nbytes)), "commands": commands}
        path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        out.append(rec)
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) |")
    print("|---|---|---|---|")
    for name in sorted(fetch, key=lambda n: -fetch[n]):
        if name in write:
            b = fetch[name] * 1024 * fetch_scale + write[name] * 1024 * write_scale
            print(f"| `{name}` | {fetch[name]:,.0f} | {write[name]:,.0f} | {b / 2**20:,.1f} MiB |")
    print(f"\nscales: fetch {fetch_scale:.4f}, write {write_scale:.4f} (from `{fk}`)")
    return out


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------

class Step:
    """Inputs, outputs and the four bound calls of one workload's step."""

    def __init__(self, moe, torch, w, d, dev, groups=None):
        self.moe, self.torch, self.w, self.dev, self.groups = moe, torch, w, dev, groups

        def up(a, bf16=False):
            if a is None:
                return None
            t = torch.from_numpy(np.ascontiguousarray(a))
            return (t.view(torch.bfloat16) if bf16 else t).to(dev)

        self.logits, self.bias = up(d["logits"]), up(d["bias"])
        self.x, self.res, self.sh = up(d["x"], True), up(d["residual"], True), up(d["shared"], True)
        self.send_rows = moe.send_rows_bound(w.T, w.k, w.E, w.capacity)
        self.main = self.output_set()

    def output_set(self):
        """Everything one step writes: routing, layout, workspace, send rows, output."""
        torch, w, dev = self.torch, self.w, self.dev
        T, H, E, k, R = w.T, w.H, w.E, w.k, w.R
        i32 = dict(dtype=torch.int32, device=dev)
        return {"idx": torch.empty((T, k), **i32),
                "wt": torch.empty((T, k), dtype=torch.float32, device=dev),
                "lay": {"expert_demand": torch.empty(E, **i32), "expert_counts": torch.empty(E, **i32),
                        "expert_offsets": torch.empty(E + 1, **i32), "dest_counts": torch.empty(R, **i32),
                        "dest_offsets": torch.empty(R + 1, **i32), "pos": torch.empty((T, k), **i32),
                        "send_src": torch.empty(T * k, **i32)},
                "ws": torch.zeros(self.moe.moe_route_dispatch_layout_workspace_size(T, E, k, R), dtype=torch.uint8,
                                  device=dev),
                "send": torch.empty((self.send_rows, H), dtype=torch.bfloat16, device=dev),
                "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev)}

    def calls(self, sp, o=None, fused=True):
        """The step's calls with every pointer bound once (as a C caller holds
        them): routing and layout in one call (moe_route_dispatch_layout: one
        launch for small batches) unless fused is False or routing is
        group-limited, then the permute and the combine."""
        o = self.main if o is None else o
        moe, lib, w = self.moe, self.moe.lib, self.w
        T, H, E, k, R, C = w.T, w.H, w.E, w.k, w.R, w.capacity
        P = lambda t: None if t is None else t.data_ptr()
        lay = o["lay"]
        logits, bias, idx, wt = P(self.logits), P(self.bias), P(o["idx"]), P(o["wt"])
        ld = [P(lay[n]) for n in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts",
                                  "dest_offsets", "pos", "send_src")]
        ws, wsn, pos = P(o["ws"]), o["ws"].numel(), P(lay["pos"])
        x, send, out, sh, res = P(self.x), P(o["send"]), P(o["out"]), P(self.sh), P(self.res)
        rows, norm, g = self.send_rows, moe.MOE_ROUTE_NORMALIZE, self.groups

        def check(name, rc):
            if rc != moe.MOE_OK:
                raise RuntimeError(f"{name}: {moe.moe_status_string(rc)}")

        if g is None:
            route = lambda: check("route", lib.moe_route_topk(logits, bias, T, E, k, norm, idx, wt, sp))
        else:
            route = lambda: check("route", lib.moe_route_topk_grouped(logits, bias, T, E, k, g[0], g[1], norm,
                                                                      idx, wt, sp))
        if fused and g is None:
            first = [("route_layout", lambda: check("route_layout", lib.moe_route_dispatch_layout(
                logits, bias, T, E, k, norm, R, C, idx, wt, *ld, ws, wsn, sp)))]
        else:
            first = [("route", route),
                     ("layout", lambda: check("layout", lib.moe_dispatch_layout(idx, T, E, k, R, C, *ld, ws, wsn,
                                                                                sp)))]
        return first + [
            ("permute", lambda: check("permute", lib.moe_dispatch_permute(x, pos, T, H, k, E, C, send, rows,
                                                                          sp))),
            ("combine", lambda: check("combine", lib.moe_combine_reduce(send, rows, pos, wt, sh, res, T, H, k, 0,
                                                                        out, sp))),
        ]


def timed(torch, stream, fn, steps, warmup=0):
    """Mean ms per call of fn over `steps` calls between two events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def per_call_ms(torch, stream, calls, steps):
    """Mean ms of each call with an event pair around every call."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        for i, (_, fn) in enumerate(calls):
            ev[s][i].record(stream)
            fn()
        ev[s][len(calls)].record(stream)
    torch.cuda.synchronize()
    return {name: statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps))
            for i, (name, _) in enumerate(calls)}


def floor_rate(moe, torch, stream, read_bytes, write_bytes, steps, warmup, stores=("nt", "plain")):
    """moe_hbm_floor timed like the step, once with each store kind in
    `stores` (non-temporal, ordinary): the faster one's mean us per launch
    and GB/s, and both times."""
    read_bytes, write_bytes = read_bytes // 16 * 16, write_bytes // 16 * 16
    src = torch.empty(max(read_bytes, 16), dtype=torch.uint8, device="cuda")
    dst = torch.empty(max(write_bytes, 16), dtype=torch.uint8, device="cuda")
    us = {}
    for kind in stores:
        ms = timed(torch, stream, lambda: moe.moe_hbm_floor(src, read_bytes, dst, write_bytes,
                                                            nt_store=kind == "nt", stream=stream),
                   steps, warmup)
        us[kind] = round(ms * 1e3, 2)
    del src, dst
    best = min(us, key=us.get)
    total = read_bytes + write_bytes
    return {"read_bytes": read_bytes, "write_bytes": write_bytes, "us": us[best],
            "GBps": round(total / (us[best] * 1e-6) / 1e9, 1), "stores": best, "us_by_stores": us}


def measure_path(moe, torch, w, args, groups=None, full=True):
    """Time one workload's step. `full` adds the spread, cold-cache and
    two-stream passes and keeps the Step for the next-row measurements."""
    log("workload", w.describe())
    t0 = time.perf_counter()
    d = synthetic.make_inputs(w, seed=0)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")
    st = Step(moe, torch, w, d, torch.device("cuda:0"), groups)
    stream = torch.cuda.current_stream()
    calls = st.calls(stream.cuda_stream)
    step = lambda: [fn() for _, fn in calls]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms_eager = timed(torch, stream, step, args.steps)
    wall_eager = (time.perf_counter() - t_wall) / args.steps
    log(f"eager: {args.steps} steps, {ms_eager * 1e3:.1f} us/step (host {wall_eager * 1e6:.1f} us/step)")
    ms_graph = None
    if args.graph:
        gstream = torch.cuda.Stream()
        gcalls = st.calls(gstream.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(gstream):
            for _, fn in gcalls:
                fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gstream):
            for _, fn in gcalls:
                fn()
        torch.cuda.synchronize()
        ms_graph = timed(torch, stream, graph.replay, args.steps, args.warmup)
        log(f"graph: {args.steps} replays, {ms_graph * 1e3:.1f} us/step")
    ms_per_step = ms_eager if ms_graph is None else ms_graph

    pc = per_call_ms(torch, stream, calls, args.steps)
    log("per call (us): " + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in pc.items()))

    lay = st.main["lay"]
    T, H, E, k = w.T, w.H, w.E, w.k
    N = int(lay["expert_offsets"][E].item())
    T_read = int((lay["pos"] >= 0).any(dim=1).sum().item())
    rw = rw_bytes(w, N, T_read, st.bias is not None)
    nbytes = {n: r + wr for n, (r, wr) in rw.items()}
    total = sum(nbytes.values())
    gbps = total / (ms_per_step * 1e-3) / 1e9
    dominant = max(("permute", "combine"), key=lambda n: pc[n])
    kname = f"{dominant}_kernel"
    achieved = nbytes[dominant] / (pc[dominant] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(kname, w.name),
                "kernel": kname, "algorithmic_bytes": nbytes[dominant],
                "avg_launch_us": round(pc[dominant] * 1e3, 2)}
    # the same step with routing and layout as two separate calls
    calls4 = st.calls(stream.cuda_stream, fused=False)
    ms_four = timed(torch, stream, lambda: [fn() for _, fn in calls4], args.steps, args.warmup)
    pc4 = per_call_ms(torch, stream, calls4, args.steps)
    res = {"workload": w.describe(), "T": T, "H": H, "E": E, "k": k, "R": w.R, "capacity": w.capacity,
           "shared_expert": w.shared, "kept_rows": N, "tokens_read": T_read, "bytes_per_step": total,
           "us_per_step": round(ms_per_step * 1e3, 2), "GBps": round(gbps, 1),
           "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
           "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
           "host_us_per_step": round(wall_eager * 1e6, 1),
           "per_call_us": {n: round(v * 1e3, 2) for n, v in pc.items()},
           "per_call_GBps": {n: round(call_bytes(nbytes, n) / (v * 1e-3) / 1e9, 1) for n, v in pc.items()},
           "four_call_step_us": round(ms_four * 1e3, 2),
           "four_call_per_call_us": {n: round(v * 1e3, 2) for n, v in pc4.items()},
           "roofline": roofline}
    if ms_graph is not None:
        res["us_per_step_eager"] = round(ms_eager * 1e3, 2)

    if not args.no_floor:
        reads = sum(r for r, _ in rw.values())
        writes = sum(wr for _, wr in rw.values())
        fl = {"step": floor_rate(moe, torch, stream, reads, writes, args.steps, args.warmup),
              "permute": floor_rate(moe, torch, stream, *rw["permute"], args.steps, args.warmup),
              "combine": floor_rate(moe, torch, stream, *rw["combine"], args.steps, args.warmup),
              "write_only": floor_rate(moe, torch, stream, 0, rw["permute"][1], args.steps, args.warmup)}
        fl["value_frac_of_floor"] = round(gbps / fl["step"]["GBps"], 4)
        fl["permute_frac_of_floor"] = round(fl["permute"]["us"] / (pc["permute"] * 1e3), 4)
        fl["combine_frac_of_floor"] = round(fl["combine"]["us"] / (pc["combine"] * 1e3), 4)
        fl["note"] = ("moe_hbm_floor: contiguous 16-byte streams of the same read and write bytes, the faster "
                      "of non-temporal and ordinary stores; write_only = the permute's write bytes alone; "
                      "*_frac_of_floor = floor time / call time; token_order_rows_us = permute and combine "
                      "with token t's replicas at rows t*k+j (dropless workloads only)")
        if st.send_rows >= T * k and N == T * k and not args.no_token_order:
            # the same row kernels and bytes with token t's replicas at rows
            # t*k .. t*k + k - 1: every write in token order, no expert grouping
            o = dict(st.main)
            o["lay"] = dict(lay, pos=torch.arange(T * k, dtype=torch.int32, device=lay["pos"].device).view(T, k))
            rows = [c for c in st.calls(stream.cuda_stream, o) if c[0] in ("permute", "combine")]
            pcs = per_call_ms(torch, stream, rows, args.steps)
            fl["token_order_rows_us"] = {n: round(v * 1e3, 2) for n, v in pcs.items()}
            step()
            torch.cuda.synchronize()
        res["synthetic_floor"] = fl
        log("synthetic floor", fl)

    load = load_balance(lay["expert_demand"].cpu().numpy(), lay["expert_counts"].cpu().numpy(),
                        lay["dest_counts"].cpu().numpy())
    res["load"] = load
    if not full:
        return res, st, d, calls
    res["_ms_eager"], res["_ms_graph"] = ms_eager, ms_graph

    # pass 3: single-step spread; pass 4: cold cache; pass 5: two batches in flight
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    bounds[0].record(stream)
    for s in range(args.steps):
        step()
        bounds[s + 1].record(stream)
    torch.cuda.synchronize()
    step_us = sorted(bounds[s].elapsed_time(bounds[s + 1]) * 1e3 for s in range(args.steps))
    pct = lambda v, q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
    res["step_us_spread"] = {q: round(pct(step_us, f), 1) for q, f in (("p10", .1), ("p50", .5), ("p90", .9))}
    log("single-step us", res["step_us_spread"])

    if not args.no_cold:
        # a read, not a write: dirty scratch lines left in the cache would be
        # written back during the step and charged to it
        scratch = torch.zeros(1 << 28, dtype=torch.int32, device=st.dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for s in range(args.steps):
            torch.amax(scratch)
            cev[s][0].record(stream)
            step()
            cev[s][1].record(stream)
        torch.cuda.synchronize()
        cold_us = sorted(a.elapsed_time(b) * 1e3 for a, b in cev)
        res["step_us_cold"] = {q: round(pct(cold_us, f), 1) for q, f in (("p10", .1), ("p50", .5), ("p90", .9))}
        del scratch
        log("cold-cache single-step us", res["step_us_cold"])

    if not args.no_pipelined:
        # step s on stream s % 2 with its own outputs: one batch's routing and
        # layout (instruction issue and latency) beside the other's permute and
        # combine (HBM)
        ref_out = st.main["out"].clone()
        sets = [st.main, st.output_set()]
        pstreams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
        pcalls = [st.calls(ps.cuda_stream, o) for ps, o in zip(pstreams, sets)]

        def run_pipelined(n):
            fork = torch.cuda.Event()
            fork.record(stream)
            for ps in pstreams:
                ps.wait_event(fork)
            for s in range(n):
                for _, fn in pcalls[s % 2]:
                    fn()
            for ps in pstreams:
                joined = torch.cuda.Event()
                joined.record(ps)
                stream.wait_event(joined)

        ms_pipe = timed(torch, stream, lambda: run_pipelined(args.steps), 1, 1) / args.steps
        pipe_equal = all(torch.equal(o["out"], ref_out) for o in sets)
        res["pipelined_two_streams"] = {
            "us_per_step": round(ms_pipe * 1e3, 1), "GBps": round(total / (ms_pipe * 1e-3) / 1e9, 1),
            "tokens_per_s": round(T / (ms_pipe * 1e-3), 1),
            "speedup_vs_one_step_at_a_time": round(ms_per_step / ms_pipe, 3),
            "outputs_bitwise_equal": pipe_equal,
            "note": "two batches in flight on two streams with their own outputs; `value` is one step at a time"}
        del sets, pcalls, ref_out
        log("two batches in flight", res["pipelined_two_streams"])
    return res, st, d, calls


def bench_regroup(moe, torch, st, stream, warmup, steps, floor=True):
    """Receive-side regroup on this GPU's share: the send buffer read as a
    receive buffer of S = R source segments with E_l local experts each
    (counts = the layout's expert counts), regrouped expert-major and back.
    Algorithmic bytes per call: layout S*E_l*4 + (E_l + S + 2)*4 + N*4;
    regroup and ungroup 2*N*H*2 + N*4."""
    w, lay, send = st.w, st.main["lay"], st.main["send"]
    S, El, H, rows = w.R, w.E // w.R, w.H, st.send_rows
    dev = send.device
    i32 = dict(dtype=torch.int32, device=dev)
    cnt = lay["expert_counts"].view(S, El)
    L = {"local_expert_offsets": torch.empty(El + 1, **i32), "source_offsets": torch.empty(S + 1, **i32),
         "recv_pos": torch.empty(rows, **i32)}
    ws = torch.empty(moe.moe_recv_regroup_workspace_size(S, El), dtype=torch.uint8, device=dev)
    grouped, back = torch.empty_like(send), torch.empty_like(send)
    n_rows = L["source_offsets"][S:]
    sp, lib, P = stream.cuda_stream, moe.lib, (lambda t: t.data_ptr())

    def check(name, rc):
        if rc != moe.MOE_OK:
            raise RuntimeError(f"{name}: {moe.moe_status_string(rc)}")

    calls = [
        ("layout", lambda: check("regroup layout", lib.moe_recv_regroup_layout(
            P(cnt), S, El, P(L["local_expert_offsets"]), P(L["source_offsets"]), P(L["recv_pos"]),
            rows, P(ws), ws.numel(), sp))),
        ("regroup", lambda: check("regroup", lib.moe_recv_regroup(
            P(send), P(L["recv_pos"]), P(n_rows), rows, H, P(grouped), sp))),
        ("ungroup", lambda: check("ungroup", lib.moe_recv_ungroup(
            P(grouped), P(L["recv_pos"]), P(n_rows), rows, H, P(back), sp))),
    ]
    us_pass = timed(torch, stream, lambda: [fn() for _, fn in calls], steps, warmup) * 1e3
    us = {n: v * 1e3 for n, v in per_call_ms(torch, stream, calls, steps).items()}
    N = int(L["source_offsets"][S].item())
    if not torch.equal(back[:N].view(torch.int16), send[:N].view(torch.int16)):
        raise RuntimeError("regroup round trip did not return the receive buffer")
    nb = {"layout": S * El * 4 + (El + S + 2) * 4 + N * 4,
          "regroup": 2 * N * H * 2 + N * 4, "ungroup": 2 * N * H * 2 + N * 4}
    gbps = {n: nb[n] / (us[n] * 1e-6) / 1e9 for n in nb}
    out = {"sources": S, "local_experts": El, "rows": N, "us_per_pass": round(us_pass, 2),
           "per_call_us": {n: round(v, 2) for n, v in us.items()},
           "per_call_GBps": {n: round(v, 1) for n, v in gbps.items()},
           "roofline": {"bound": "hbm", "kernel": "regroup_rows_kernel", "achieved": round(gbps["regroup"], 1),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps["regroup"] / HBM_PEAK_GBPS, 4),
                        "traffic": stored_traffic("regroup_rows_kernel", w.name),
                        "algorithmic_bytes": nb["regroup"]}}
    if floor:
        # the synthetic floor for one direction's bytes (rows + recv_pos read, rows written)
        fl = floor_rate(moe, torch, stream, N * H * 2 + N * 4, N * H * 2, steps, warmup)
        out["synthetic_floor"] = fl
        out["frac_of_floor"] = {n: round(fl["us"] / us[n], 4) for n in ("regroup", "ungroup")}
    log("regroup", out)
    return out


def bench_fp8(moe, torch, st, calls, nbytes, stream, warmup, steps, floor=True):
    """The step with the FP8 dispatch payload: route -> layout ->
    moe_dispatch_permute_fp8 -> combine. The expert is the identity on the
    decoded rows: y = moe_fp8_dequant(send) is made once, before timing (a
    real expert matmul reads the FP8 rows itself and writes bf16 y).
    Algorithmic bytes of the FP8 permute: T*k*4 + T_read*H*2 + N*row_bytes."""
    w, lay = st.w, st.main["lay"]
    T, H, E, k, C, rows = w.T, w.H, w.E, w.k, w.capacity, st.send_rows
    dev = st.x.device
    rb = moe.moe_fp8_row_bytes(H)
    send8 = torch.empty((rows, rb), dtype=torch.uint8, device=dev)
    y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    sp, lib = stream.cuda_stream, moe.lib
    P = lambda t: None if t is None else t.data_ptr()
    x, pos, wt, sh, res, s8, yp, op = (P(st.x), P(lay["pos"]), P(st.main["wt"]), P(st.sh), P(st.res),
                                       P(send8), P(y), P(out))

    def check(name, rc):
        if rc != moe.MOE_OK:
            raise RuntimeError(f"{name}: {moe.moe_status_string(rc)}")

    fcalls = [c for c in calls if c[0] not in ("permute", "combine")] + [
        ("permute_fp8", lambda: check("permute_fp8", lib.moe_dispatch_permute_fp8(
            x, pos, T, H, k, E, C, s8, rows, sp))),
        ("combine", lambda: check("combine", lib.moe_combine_reduce(
            yp, rows, pos, wt, sh, res, T, H, k, 0, op, sp))),
    ]
    for _, fn in fcalls[:-1]:
        fn()
    check("fp8 dequant", lib.moe_fp8_dequant(s8, P(lay["expert_offsets"][E:]), rows, H, yp, sp))
    ms_step = timed(torch, stream, lambda: [fn() for _, fn in fcalls], steps, warmup)
    us = {n: v * 1e3 for n, v in per_call_ms(torch, stream, fcalls, steps).items()}
    N = int(lay["expert_offsets"][E].item())
    T_read = int((lay["pos"] >= 0).any(dim=1).sum().item())
    nb = dict(nbytes)
    del nb["permute"]
    nb["permute_fp8"] = T * k * 4 + T_read * H * 2 + N * rb
    total = sum(nb.values())
    gbps_p = nb["permute_fp8"] / (us["permute_fp8"] * 1e-6) / 1e9
    report = {"row_bytes": rb, "bytes_per_step": total, "us_per_step": round(ms_step * 1e3, 2),
              "GBps": round(total / (ms_step * 1e-3) / 1e9, 1), "tokens_per_s": round(T / (ms_step * 1e-3), 1),
              "per_call_us": {n: round(v, 2) for n, v in us.items()},
              "roofline": {"bound": "hbm", "kernel": "permute_fp8_kernel", "achieved": round(gbps_p, 1),
                           "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps_p / HBM_PEAK_GBPS, 4),
                           "traffic": stored_traffic("permute_fp8_kernel", w.name),
                           "algorithmic_bytes": nb["permute_fp8"]},
              "note": "send rows hold E4M3 codes plus one scale byte per 32 values; combine reads the "
                      "identity expert's bf16 output, decoded once before timing"}
    if floor:
        # the synthetic floor for the FP8 permute's own read and write bytes
        fl = floor_rate(moe, torch, stream, T * k * 4 + T_read * H * 2, N * rb, steps, warmup)
        report["synthetic_floor"] = fl
        report["permute_fp8_frac_of_floor"] = round(fl["us"] / us["permute_fp8"], 4)
    log("fp8 dispatch", report)
    return report


def token_ready_profile(cnt, pos, self_rank=0, band_rows=128, marks=(0.5, 0.75, 0.9, 0.99)):
    """When each token's rows are all computed in the tile-signalled GEMM's
    work order: bands of 128 rows of each (source, local expert) block, the
    sources remote-first (self_rank + 1, ..., self_rank last), experts
    ascending. Returns the share of tokens with a kept row whose last band is
    among the first q of all bands, for each q in marks: the part of the
    combine that could start before the GEMM ends."""
    S, El = cnt.shape
    starts = np.concatenate([[0], np.cumsum(cnt.ravel())])
    band_of_row = np.empty(int(starts[-1]), np.int64)
    b = 0
    for s in [(self_rank + i) % S for i in range(1, S + 1)]:
        for l in range(El):
            n, r0 = int(cnt[s, l]), int(starts[s * El + l])
            band_of_row[r0:r0 + n] = b + np.arange(n) // band_rows
            b += (n + band_rows - 1) // band_rows
    kept = pos >= 0
    has = kept.any(axis=1)
    if b == 0 or not has.any():
        return {"bands": b, "tokens": 0}
    last = np.where(kept, band_of_row[np.where(kept, pos, 0)], -1).max(axis=1)[has]
    frac = (last + 1) / b
    return {"bands": b, "tokens": int(has.sum()),
            "share_ready_by_band_share": {str(q): round(float((frac <= q).mean()), 4) for q in marks}}


def bench_tile_return(moe, torch, st, stream, warmup, steps, seed=0):
    """Tile-signalled return on this GPU's share: the send buffer read as S
    source segments of E_l local experts goes through a stand-in expert (one
    H x H linear map per local expert, MFMA bf16), and the results return to
    the sources' buffer. Timed: the GEMM alone, the GEMM then a copy of y to
    ret (the return starting after the GEMM), and the signalled launch with
    16, 24 and 32 dedicated consumer blocks (of one block per CU) and with
    none (producers return their own tasks). FLOPs per GEMM: 2 * N * H * H."""
    w, lay, send = st.w, st.main["lay"], st.main["send"]
    S, El, H, rows = w.R, w.E // w.R, w.H, st.send_rows
    dev = send.device
    cnt = lay["expert_counts"].view(S, El)
    W = torch.from_numpy(synthetic.make_expert_weights(El, H, H, seed).view(np.int16)).to(dev).view(torch.bfloat16)
    ws = torch.empty(moe.moe_expert_linear_workspace_size(S, El, rows), dtype=torch.uint8, device=dev)
    y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    ret = torch.empty_like(y)
    gemm = lambda: moe.moe_expert_linear(send, cnt, W, y=y, workspace=ws)
    us = {"gemm": timed(torch, stream, gemm, steps, warmup) * 1e3,
          "gemm_then_copy": timed(torch, stream, lambda: (gemm(), ret.copy_(y)), steps, warmup) * 1e3}
    status = {}
    for consumers in CONSUMER_COUNTS:
        key = f"signalled_consumers_{consumers}"
        us[key] = timed(torch, stream, lambda: moe.moe_expert_linear_return(
            send, cnt, W, 0, consumers, 2, y=y, ret=ret, workspace=ws), steps, warmup) * 1e3
        status[key] = int(ws[:4].view(torch.int32).item())
    if any(status.values()):
        raise RuntimeError(f"tile-signalled return reported status {status}")
    N = int(lay["expert_offsets"][-1].item())
    if not torch.equal(ret[:N].view(torch.int16), y[:N].view(torch.int16)):
        raise RuntimeError("returned rows differ from the expert output")
    flops = 2.0 * N * H * H
    tflops = flops / (us["gemm"] * 1e-6) / 1e12
    best = min((k for k in us if k.startswith("signalled_")), key=lambda k: us[k])
    out = {"workload": w.name, "rows": N, "sources": S, "local_experts": El, "H": H,
           "per_call_us": {k: round(v, 1) for k, v in us.items()},
           "signalled_vs_sequential": round(us["gemm_then_copy"] / us[best], 3),
           "best_signalled": best,
           "roofline": {"bound": "mfma", "kernel": "expert_linear_kernel", "achieved": round(tflops, 1),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "flops": flops},
           "token_ready_profile": token_ready_profile(cnt.cpu().numpy(), lay["pos"].cpu().numpy()),
           "note": "stand-in expert: one bf16 H x H linear map per local expert; band_group 2"}
    log("tile-signalled return", out)
    return out


def main(argv=None):
    args = parse(argv)
    if args.summarize:
        summarize(args.summarize)
        return
    if args.write_traffic:
        # the counter runs as made from the repository root, into the two
        # directories this call reads
        cmds = [f"rocprofv3 --pmc {c} -d {d} -o run --output-format csv -- python3 bench.py --workload "
                f"{args.workload} --steps 2 --warmup 1 --also '' --no-cpu-baseline --no-tile-return --no-floor "
                f"--calibrate"
                for c, d in (("FETCH_SIZE", args.write_traffic[0]), ("WRITE_SIZE", args.write_traffic[1]))]
        write_traffic(args.write_traffic[0], args.write_traffic[1], workload_by_name(args.workload).name, cmds)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no inter-GPU exchange "
              "(the R destinations are partitions of one HBM buffer); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_route_topk_amd as moe

    torch.cuda.set_device(torch.device("cuda:0"))
    stream = torch.cuda.current_stream()
    w = workload_by_name(args.workload)
    groups = None if args.route_groups is None else tuple(int(v) for v in args.route_groups.split(","))
    r, st, d, calls = measure_path(moe, torch, w, args, groups, full=True)
    ms_per_step = r.pop("_ms_graph") or r["_ms_eager"]
    ms_eager = r.pop("_ms_eager")
    nbytes = algorithmic_bytes(w, r["kept_rows"], r["tokens_read"], st.bias is not None)

    next_rows = {}
    if not args.no_fp8 and w.H % 32 == 0:
        next_rows["fp8_dispatch"] = bench_fp8(moe, torch, st, calls, nbytes, stream, args.warmup, args.steps,
                                              floor=not args.no_floor)
    if not args.no_regroup and w.R >= 2:
        next_rows["recv_regroup"] = bench_regroup(moe, torch, st, stream, args.warmup, args.steps,
                                                  floor=not args.no_floor)
    if not args.no_tile_return and w.R >= 2 and w.H % 128 == 0:
        next_rows["tile_signalled_return"] = bench_tile_return(moe, torch, st, stream, args.warmup, args.steps)
    cpu_d = d
    del st, calls

    workloads = {}
    for name in [n for n in args.also.split(",") if n]:
        wx = workload_by_name(name)
        if wx.name == w.name:
            continue
        rx, stx, _, cx = measure_path(moe, torch, wx, args, groups, full=False)
        if wx.name in PREFILL and not args.no_fp8 and wx.H % 32 == 0:
            nbx = algorithmic_bytes(wx, rx["kept_rows"], rx["tokens_read"], stx.bias is not None)
            rx["fp8_dispatch"] = bench_fp8(moe, torch, stx, cx, nbx, stream, args.warmup, args.steps,
                                               floor=not args.no_floor)
        if wx.name in PREFILL and not args.no_tile_return and wx.R >= 2 and wx.H % 128 == 0:
            rx["tile_signalled_return"] = bench_tile_return(moe, torch, stx, stream, args.warmup, args.steps)
        workloads[wx.name] = rx
        del stx, cx
        torch.cuda.empty_cache()
    if "tile_signalled_return" in next_rows:
        by = {w.name: next_rows["tile_signalled_return"]["signalled_vs_sequential"]}
        by.update({n: v["tile_signalled_return"]["signalled_vs_sequential"]
                   for n, v in workloads.items() if "tile_signalled_return" in v})
        next_rows["tile_signalled_return"]["signalled_vs_sequential_by_workload"] = by

    calibration = None
    if args.calibrate:
        # the floor kernel as a plain 1 GiB copy: the launch counter runs are scaled by
        calibration = floor_rate(moe, torch, stream, FLOOR_CALIBRATION_BYTES, FLOOR_CALIBRATION_BYTES, 3, 1,
                                 stores=("nt",))
        log("calibration copy", calibration)

    result = {
        "metric": "dispatch+combine HBM GB/s (% of MI355X peak) and tokens/s, 1 GPU",
        "value": r["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["workload"] + ("" if groups is None else
                                                f", at most {groups[1]} of {groups[0]} expert groups per token"),
                   "T": w.T, "H": w.H, "E": w.E, "k": w.k, "R": w.R,
                   "capacity": w.capacity, "shared_expert": w.shared, "kept_rows": r["kept_rows"],
                   "tokens_read": r["tokens_read"], "bytes_per_step": r["bytes_per_step"],
                   "parallelism": "single GPU (R logical destinations)"},
        "pct_of_hbm_peak": r["pct_of_hbm_peak"],
        "tokens_per_s": r["tokens_per_s"],
        "per_call_us": r["per_call_us"],
        "timing": "one HIP graph replay per step (four launches)" if args.graph else "eager launches",
        "ms_per_step_eager": round(ms_eager, 5),
        "host_us_per_step": r["host_us_per_step"],
        "per_call_note": ("second pass of the same K steps with an event pair around every call; "
                          "route_layout is moe_route_dispatch_layout (one launch when T*k <= 4096 and "
                          "E <= 512, else the routing and layout kernels)"),
        "four_call_step_us": r["four_call_step_us"],
        "four_call_per_call_us": r["four_call_per_call_us"],
        "per_call_GBps": r["per_call_GBps"],
        "step_us_spread": r.get("step_us_spread"),
        "step_us_spread_note": "third pass of K steps with one event between consecutive steps",
        "step_us_cold": r.get("step_us_cold"),
        "step_us_cold_note": ("fourth pass of K steps, each after a read of a 1 GiB scratch buffer "
                              "(outside its event pair) that evicts the 256 MB Infinity Cache"),
        "roofline": r["roofline"],
    }
    if "synthetic_floor" in r:
        result["synthetic_floor"] = r["synthetic_floor"]
    if workloads:
        result["workloads"] = workloads
        result["workloads_note"] = ("the other workloads, measured as `value` is (eager, K steps after W "
                                    "warm-up steps, per-call event pairs in a second pass)")
    if next_rows:
        result["next_rows"] = next_rows
    result["load"] = r["load"]
    if "pipelined_two_streams" in r:
        result["pipelined_two_streams"] = r["pipelined_two_streams"]
    if calibration:
        result["floor_calibration_copy"] = calibration

    if not args.no_cpu_baseline:
        log("cpu baseline: timing the C oracle on the same host arrays")
        sec, reps = cpu_baseline(w, cpu_d, args.cpu_seconds)
        model, affinity = host_cpu()
        result["cpu_baseline"] = {
            "value": round(r["bytes_per_step"] / sec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the full {w.name} batch (T={w.T}), {reps} rep(s), median {sec:.2f}s per pass; "
                      f"single-threaded C oracle on {model}",
            "tokens_per_s": round(w.T / sec, 1),
            "host": {"cpu_model": model, "affinity_cores": affinity, "threads_used": 1},
        }
        log("cpu baseline", result["cpu_baseline"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
