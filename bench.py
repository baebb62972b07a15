"""Benchmark of the MoE dispatch/combine core on one MI355X.

One step = the whole path over one synthetic batch already resident in HBM:
moe_route_topk -> moe_dispatch_layout -> moe_dispatch_permute ->
moe_combine_reduce (the expert is the identity: combine reads the send
buffer). W untimed warm-up steps, then exactly K timed steps between
device synchronisations with HIP events only at the two ends (an event
between calls leaves the GPU idle for a few microseconds). The steps are
eager launches; --graph times replays of a HIP graph that holds the four
launches instead (on MI355X a replay cost 22 us where the four eager
launches of the decode workload cost 16 us, so eager is the default). A second pass of
K steps records an event pair around every call, on the stream the kernels
run on, for the per-call durations and the roofline of the dominant kernel.

Prints ONE JSON line on stdout. `value` is algorithmic HBM bytes per step /
step time (GB/s); tokens/s and the fraction of the 8 TB/s peak ride along.
Algorithmic bytes count every array each call must read once and write once,
for kept rows only:
  route    T*E*4 (+E*4 bias) + 2*T*k*4
  layout   2*T*k*4 + N*4 + (3E + 2R + 2)*4
  permute  T*k*4 + T_read*H*2 + N*H*2
  combine  2*T*k*4 + N*H*2 + T*H*2*(residual + shared) + T*H*2
with N kept rows and T_read tokens that have at least one kept replica (both
read from the path's own outputs after the timed region).

After the path, three further measurements are reported under "next_rows",
none part of `value`:
  * the same step with the FP8 dispatch payload (moe_dispatch_permute_fp8 in
    place of the bf16 permute);
  * the receive-side regroup on the same buffers (the send buffer read as R
    source segments);
  * the tile-signalled return: a stand-in expert GEMM on those segments whose
    tiles are returned as they finish, against the GEMM then a copy.

Alongside: the spread of single-step times (a third pass with one event
between steps); the same spread from a cold cache (a fourth pass, each step
after a 1 GiB scratch read that evicts the Infinity Cache); a fifth pass
with two batches in flight on two streams, each with its own outputs, whose
results must equal a step on its own bit for bit ("pipelined_two_streams");
the load imbalance read from the layout's own counts ("load"); and a
synthetic floor -- a device-to-device copy moving the step's byte count,
half read and half written, timed like the step -- as the achievable HBM
rate for the same volume.

The CPU-baseline leg times the plain C oracle on the same host arrays:
whole passes on one core for about --cpu-seconds, median pass.
"""

from __future__ import annotations

import argparse
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
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "combine_kernel": "combine_route_topk_amd/csrc/combine.hip",
    "permute_kernel": "combine_route_topk_amd/csrc/permute.hip",
    "permute_fp8_kernel": "combine_route_topk_amd/csrc/fp8.hip",
    "regroup_rows_kernel": "combine_route_topk_amd/csrc/regroup.hip",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="fine_grained",
                   help="one of " + ", ".join(w.name for w in synthetic.WORKLOADS.values()))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time replays of a captured HIP graph of the step instead of eager launches "
                        "(on MI355X with ROCm 7 a replay costs more than four eager launches)")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cold-cache pass (each step after a 1 GiB scratch read)")
    p.add_argument("--no-floor", action="store_true",
                   help="skip the synthetic floor (a device-to-device copy of the step's bytes)")
    p.add_argument("--no-pipelined", action="store_true",
                   help="skip the pass with two batches in flight on two streams (reported beside value)")
    p.add_argument("--no-fp8", action="store_true",
                   help="skip the FP8-payload step measurement (reported under next_rows)")
    p.add_argument("--no-tile-return", action="store_true",
                   help="skip the tile-signalled return measurement (reported under next_rows)")
    p.add_argument("--no-regroup", action="store_true",
                   help="skip the receive-side regroup measurement (reported under next_rows)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="rough CPU time budget of the oracle baseline")
    p.add_argument("--route-groups", default=None, metavar="G,M",
                   help="route with moe_route_topk_grouped: at most M of G expert groups per token")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run a plain copy kernel of this size (for counter calibration)")
    return p.parse_args()


def workload_by_name(name):
    for i, w in synthetic.WORKLOADS.items():
        if name in (w.name, str(i)):
            return w
    raise SystemExit(f"unknown workload {name}")


def algorithmic_bytes(w, N, T_read, has_bias):
    T, H, E, k, R = w.T, w.H, w.E, w.k, w.R
    dense = 1 + (1 if w.residual else 0) + (1 if w.shared else 0)   # out + residual + shared
    return {
        "route": T * E * 4 + (E * 4 if has_bias else 0) + 2 * T * k * 4,
        "layout": 2 * T * k * 4 + N * 4 + (3 * E + 2 * R + 2) * 4,
        "permute": T * k * 4 + T_read * H * 2 + N * H * 2,
        "combine": 2 * T * k * 4 + N * H * 2 + T * H * 2 * dense,
    }


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


def bench_regroup(moe, torch, lay, send, S, El, H, rows, stream, warmup, steps, workload):
    """Receive-side regroup on this GPU's share: the send buffer read as a
    receive buffer of S source segments with El local experts each (counts =
    the layout's expert counts), regrouped expert-major and back. Per-call
    event pairs; algorithmic bytes per call:
      layout   S*El*4 + (El + S + 2)*4 + N*4
      regroup  N*H*2 read + N*H*2 write + N*4
      ungroup  the same."""
    dev = send.device
    i32 = dict(dtype=torch.int32, device=dev)
    cnt = lay["expert_counts"].view(S, El)
    L = {"local_expert_offsets": torch.empty(El + 1, **i32), "source_offsets": torch.empty(S + 1, **i32),
         "recv_pos": torch.empty(rows, **i32)}
    ws = torch.empty(moe.moe_recv_regroup_workspace_size(S, El), dtype=torch.uint8, device=dev)
    grouped = torch.empty_like(send)
    back = torch.empty_like(send)
    n_rows = L["source_offsets"][S:]
    sp = stream.cuda_stream
    lib, P = moe.lib, (lambda t: t.data_ptr())

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
    for _ in range(warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    beg, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    beg.record(stream)
    for _ in range(steps):
        for _, fn in calls:
            fn()
    end.record(stream)
    torch.cuda.synchronize()
    us_pass = beg.elapsed_time(end) / steps * 1e3
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for s in range(steps):
        for i, (_, fn) in enumerate(calls):
            ev[s][i].record(stream)
            fn()
        ev[s][len(calls)].record(stream)
    torch.cuda.synchronize()
    us = {name: statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) * 1e3
          for i, (name, _) in enumerate(calls)}
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
                        "traffic": stored_traffic("regroup_rows_kernel", workload),
                        "algorithmic_bytes": nb["regroup"]}}
    log("regroup", out)
    return out


def bench_fp8(moe, torch, calls, lay, x, wt, sh, res, T, H, E, k, send_rows, nbytes, stream,
              warmup, steps, workload):
    """The step with the FP8 dispatch payload: route -> layout ->
    moe_dispatch_permute_fp8 -> combine. The expert is the identity on the
    decoded rows: y = moe_fp8_dequant(send) is made once, before timing (a
    real expert matmul reads the FP8 rows itself and writes bf16 y).
    Algorithmic bytes of the FP8 permute: T*k*4 + T_read*H*2 + N*row_bytes."""
    dev = x.device
    rb = moe.moe_fp8_row_bytes(H)
    send8 = torch.empty((send_rows, rb), dtype=torch.uint8, device=dev)
    y = torch.empty((send_rows, H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    sp = stream.cuda_stream
    lib, P = moe.lib, (lambda t: None if t is None else t.data_ptr())

    def check(name, rc):
        if rc != moe.MOE_OK:
            raise RuntimeError(f"{name}: {moe.moe_status_string(rc)}")

    fcalls = calls[:2] + [
        ("permute_fp8", lambda: check("permute_fp8", lib.moe_dispatch_permute_fp8(
            P(x), P(lay["pos"]), T, H, k, P(send8), send_rows, sp))),
        ("combine", lambda: check("combine", lib.moe_combine_reduce(
            P(y), send_rows, P(lay["pos"]), P(wt), P(sh), P(res), T, H, k, 0, P(out), sp))),
    ]
    for _, fn in fcalls[:3]:
        fn()
    check("fp8 dequant", lib.moe_fp8_dequant(P(send8), P(lay["expert_offsets"][E:]), send_rows, H,
                                             P(y), sp))
    for _ in range(warmup):
        for _, fn in fcalls:
            fn()
    torch.cuda.synchronize()
    beg, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    beg.record(stream)
    for _ in range(steps):
        for _, fn in fcalls:
            fn()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = beg.elapsed_time(end) / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fcalls) + 1)] for _ in range(steps)]
    for s in range(steps):
        for i, (_, fn) in enumerate(fcalls):
            ev[s][i].record(stream)
            fn()
        ev[s][len(fcalls)].record(stream)
    torch.cuda.synchronize()
    us = {name: statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) * 1e3
          for i, (name, _) in enumerate(fcalls)}
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
                        "traffic": stored_traffic("permute_fp8_kernel", workload),
                        "algorithmic_bytes": nb["permute_fp8"]},
           "note": "send rows hold E4M3 codes plus one scale byte per 32 values; combine reads the "
                   "identity expert's bf16 output, decoded once before timing"}
    log("fp8 dispatch", report)
    return report


MFMA_BF16_PEAK_TFLOPS = 2500.0
CONSUMER_COUNTS = (16, 24, 32, 0)   # dedicated consumer blocks tried by the tile-signalled return


def bench_tile_return(moe, torch, lay, send, S, El, H, rows, stream, warmup, steps, seed=0):
    """Tile-signalled return on this GPU's share: the send buffer read as S
    source segments of El local experts goes through a stand-in expert (one
    H x H linear map per local expert, MFMA bf16), and the results return to
    the sources' buffer. Timed: the GEMM alone, the GEMM then a copy of y to
    ret (the return starting after the GEMM), and the signalled launch with
    16, 24 and 32 dedicated consumer blocks (of one block per CU) and with
    none (producers return their own tasks). FLOPs per GEMM: 2 * N * H * H."""
    dev = send.device
    cnt = lay["expert_counts"].view(S, El)
    W = torch.from_numpy(synthetic.make_expert_weights(El, H, H, seed).view(np.int16)).to(dev).view(torch.bfloat16)
    ws = torch.empty(moe.moe_expert_linear_workspace_size(S, El, rows), dtype=torch.uint8, device=dev)
    y = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    ret = torch.empty_like(y)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    gemm = lambda: moe.moe_expert_linear(send, cnt, W, y=y, workspace=ws)
    us = {"gemm": timed(gemm), "gemm_then_copy": timed(lambda: (gemm(), ret.copy_(y)))}
    status = {}
    for consumers in CONSUMER_COUNTS:
        key = f"signalled_consumers_{consumers}"
        us[key] = timed(lambda: moe.moe_expert_linear_return(send, cnt, W, 0, consumers, 2, y=y, ret=ret,
                                                             workspace=ws))
        status[key] = int(ws[:4].view(torch.int32).item())
    if any(status.values()):
        raise RuntimeError(f"tile-signalled return reported status {status}")
    N = int(lay["expert_offsets"][-1].item())
    if not torch.equal(ret[:N].view(torch.int16), y[:N].view(torch.int16)):
        raise RuntimeError("returned rows differ from the expert output")
    flops = 2.0 * N * H * H
    tflops = flops / (us["gemm"] * 1e-6) / 1e12
    best = min((k for k in us if k.startswith("signalled_")), key=lambda k: us[k])
    out = {"rows": N, "sources": S, "local_experts": El, "H": H,
           "per_call_us": {k: round(v, 1) for k, v in us.items()},
           "signalled_vs_sequential": round(us["gemm_then_copy"] / us[best], 3),
           "best_signalled": best,
           "roofline": {"bound": "mfma", "kernel": "expert_linear_kernel", "achieved": round(tflops, 1),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "flops": flops},
           "note": "stand-in expert: one bf16 H x H linear map per local expert; band_group 2"}
    log("tile-signalled return", out)
    return out


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


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no inter-GPU exchange "
              "(the R destinations are partitions of one HBM buffer); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_route_topk_amd as moe

    w = workload_by_name(args.workload)
    log("workload", w.describe())
    t0 = time.perf_counter()
    d = synthetic.make_inputs(w, seed=0)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a, bf16=False):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)

    logits, bias = up(d["logits"]), up(d["bias"])
    x, res, sh = up(d["x"], True), up(d["residual"], True), up(d["shared"], True)
    T, H, E, k, R, C = w.T, w.H, w.E, w.k, w.R, w.capacity
    send_rows = T * k if C < 0 else min(T * k, E * C)
    i32 = dict(dtype=torch.int32, device=dev)

    def output_set():
        """Everything one step writes: routing, layout, workspace, send rows, output."""
        return {"idx": torch.empty((T, k), **i32),
                "wt": torch.empty((T, k), dtype=torch.float32, device=dev),
                "lay": {"expert_demand": torch.empty(E, **i32), "expert_counts": torch.empty(E, **i32),
                        "expert_offsets": torch.empty(E + 1, **i32), "dest_counts": torch.empty(R, **i32),
                        "dest_offsets": torch.empty(R + 1, **i32), "pos": torch.empty((T, k), **i32),
                        "send_src": torch.empty(T * k, **i32)},
                "ws": torch.empty(max(moe.moe_layout_workspace_size(T, E, k, R), 16), dtype=torch.uint8,
                                  device=dev),
                "send": torch.empty((send_rows, H), dtype=torch.bfloat16, device=dev),
                "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev)}

    main_set = output_set()
    idx, wt, lay, ws = main_set["idx"], main_set["wt"], main_set["lay"], main_set["ws"]
    send, out = main_set["send"], main_set["out"]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    groups = None if args.route_groups is None else tuple(int(v) for v in args.route_groups.split(","))
    lib = moe.lib
    P = lambda t: None if t is None else t.data_ptr()

    def check(name, rc):
        if rc != moe.MOE_OK:
            raise RuntimeError(f"{name}: {moe.moe_status_string(rc)}")

    def make_calls(sp, o=main_set):
        idx, wt, lay, ws, send, out = o["idx"], o["wt"], o["lay"], o["ws"], o["send"], o["out"]
        return [
            ("route", lambda: check("route", lib.moe_route_topk(
                P(logits), P(bias), T, E, k, moe.MOE_ROUTE_NORMALIZE, P(idx), P(wt), sp))
             if groups is None else check("route", lib.moe_route_topk_grouped(
                P(logits), P(bias), T, E, k, groups[0], groups[1], moe.MOE_ROUTE_NORMALIZE, P(idx),
                P(wt), sp))),
            ("layout", lambda: check("layout", lib.moe_dispatch_layout(
                P(idx), T, E, k, R, C, P(lay["expert_demand"]), P(lay["expert_counts"]),
                P(lay["expert_offsets"]), P(lay["dest_counts"]), P(lay["dest_offsets"]),
                P(lay["pos"]), P(lay["send_src"]), P(ws), ws.numel(), sp))),
            ("permute", lambda: check("permute", lib.moe_dispatch_permute(
                P(x), P(lay["pos"]), T, H, k, P(send), send_rows, sp))),
            ("combine", lambda: check("combine", lib.moe_combine_reduce(
                P(send), send_rows, P(lay["pos"]), P(wt), P(sh), P(res), T, H, k, 0, P(out), sp))),
        ]

    calls = make_calls(sp)

    def step(evs=None):
        for i, (_, fn) in enumerate(calls):
            if evs is not None:
                evs[i].record(stream)
            fn()
        if evs is not None:
            evs[len(calls)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # pass 1 (the measurement): K steps between synchronisations, with events
    # only at the two ends -- an event between calls costs the GPU a few us
    # of idle time, which would be charged to the path. With --graph each step
    # is one replay of a HIP graph holding the four launches (captured once,
    # outside the timed region); the eager loop is timed and reported anyway.
    def timed_steps(run_one):
        t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        t_beg.record(stream)
        for _ in range(args.steps):
            run_one()
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_beg.elapsed_time(t_end) / args.steps, (time.perf_counter() - t_wall) / args.steps

    ms_eager, wall_eager = timed_steps(step)
    log(f"eager: {args.steps} steps, {ms_eager * 1e3:.1f} us/step (wall {wall_eager * 1e6:.1f} us/step)")
    graph = None
    if args.graph:
        gstream = torch.cuda.Stream()
        gcalls = make_calls(gstream.cuda_stream)
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
        for _ in range(args.warmup):
            graph.replay()
        ms_graph, wall_graph = timed_steps(graph.replay)
        log(f"graph: {args.steps} replays, {ms_graph * 1e3:.1f} us/step (wall {wall_graph * 1e6:.1f} us/step)")
    ms_per_step = ms_eager if graph is None else ms_graph
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step")

    # pass 2: K more steps with an event pair around every call, for the
    # per-call durations and the roofline of the dominant kernel
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    per_call_ms = {name: statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps))
                   for i, (name, _) in enumerate(calls)}
    log("per call (us): " + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in per_call_ms.items()))

    # pass 3: K more steps with one event between consecutive steps, for the
    # spread of single-step times (median, p10, p90)
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    bounds[0].record(stream)
    for s in range(args.steps):
        step()
        bounds[s + 1].record(stream)
    torch.cuda.synchronize()
    step_us = sorted(bounds[s].elapsed_time(bounds[s + 1]) * 1e3 for s in range(args.steps))
    pct = lambda q: step_us[min(len(step_us) - 1, int(round(q * (len(step_us) - 1))))]
    spread = {"p10": round(pct(0.1), 1), "p50": round(pct(0.5), 1), "p90": round(pct(0.9), 1)}
    log("single-step us", spread)

    # pass 4: K more steps from a cold cache -- before each, outside its
    # event pair, a read of a 1 GiB scratch buffer pushes the step's arrays
    # out of the 256 MB Infinity Cache. A read, not a write: dirty scratch
    # lines left in the cache would be written back during the step and
    # charged to it (36 us on fine_grained, measured).
    cold = None
    if not args.no_cold:
        scratch = torch.zeros(1 << 28, dtype=torch.int32, device=dev)
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
        cp = lambda q: cold_us[min(len(cold_us) - 1, int(round(q * (len(cold_us) - 1))))]
        cold = {"p10": round(cp(0.1), 1), "p50": round(cp(0.5), 1), "p90": round(cp(0.9), 1)}
        del scratch
        log("cold-cache single-step us", cold)

    # pass 5: K more steps with two batches in flight. Step s runs on stream
    # s % 2 with its own outputs, so the routing and layout of one batch
    # (bound by instruction issue and latency) can run beside the other's
    # permute and combine (bound by HBM). Reported beside `value`, which stays
    # the time of one step on its own. (Making each permute wait for the
    # previous combine, so that only routing and layout overlap, measured
    # slower: the cross-stream waits cost more than they saved.)
    ms_pipe, pipe_equal = None, None
    if not args.no_pipelined:
        ref_out = out.clone()                     # a step on its own, from the passes above
        sets = [main_set, output_set()]
        pstreams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
        pcalls = [make_calls(ps.cuda_stream, o) for ps, o in zip(pstreams, sets)]

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

        torch.cuda.synchronize()
        run_pipelined(max(args.warmup, 2))
        torch.cuda.synchronize()
        pb, pe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pb.record(stream)
        run_pipelined(args.steps)
        pe.record(stream)
        torch.cuda.synchronize()
        ms_pipe = pb.elapsed_time(pe) / args.steps
        pipe_equal = all(torch.equal(o["out"], ref_out) for o in sets)
        del sets, pcalls, ref_out
        log(f"two batches in flight: {ms_pipe * 1e3:.1f} us/step, outputs bitwise equal: {pipe_equal}")

    # bookkeeping from the path's own outputs (outside the timed region)
    N = int(lay["expert_offsets"][E].item())
    T_read = int((lay["pos"] >= 0).any(dim=1).sum().item())
    load = load_balance(lay["expert_demand"].cpu().numpy(), lay["expert_counts"].cpu().numpy(),
                        lay["dest_counts"].cpu().numpy())
    log("load", load)
    nbytes = algorithmic_bytes(w, N, T_read, bias is not None)
    total = sum(nbytes.values())
    gbps = total / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = T / (ms_per_step * 1e-3)

    dominant = max(("permute", "combine"), key=lambda n: per_call_ms[n])
    kname = f"{dominant}_kernel"
    achieved = nbytes[dominant] / (per_call_ms[dominant] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(kname, w.name),
                "kernel": kname, "algorithmic_bytes": nbytes[dominant],
                "avg_launch_us": round(per_call_ms[dominant] * 1e3, 2)}

    fp8 = None if args.no_fp8 or H % 32 else bench_fp8(
        moe, torch, calls, lay, x, wt, sh, res, T, H, E, k, send_rows, nbytes, stream,
        args.warmup, args.steps, w.name)
    tile_return = None if args.no_tile_return or R < 2 or H % 128 else bench_tile_return(
        moe, torch, lay, send, R, E // R, H, send_rows, stream, args.warmup, args.steps)
    regroup = None if args.no_regroup or R < 2 else bench_regroup(
        moe, torch, lay, send, R, E // R, H, send_rows, stream, args.warmup, args.steps, w.name)

    # synthetic floor: a device-to-device copy moving the step's byte count
    # (half read, half written), timed like the step
    floor = None
    if not args.no_floor:
        half = total // 2
        src = torch.empty(half, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        floor_ms = e0.elapsed_time(e1) / args.steps
        floor = {"bytes": 2 * half, "us": round(floor_ms * 1e3, 1),
                 "GBps": round(2 * half / (floor_ms * 1e-3) / 1e9, 1)}
        floor["value_frac_of_floor"] = round(gbps / floor["GBps"], 4)
        del src, dst
        log("synthetic floor", floor)

    copy_probe = None
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 2
        a = torch.randn(n, device=dev).to(torch.bfloat16)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            torch.neg(a, out=b)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        copy_probe = {"bytes_per_launch": 2 * a.numel() * 2, "avg_launch_us": round(ms * 1e3, 2),
                      "GBps": round(2 * a.numel() * 2 / (ms * 1e-3) / 1e9, 1)}
        log("copy probe", copy_probe)

    result = {
        "metric": "dispatch+combine HBM GB/s (% of MI355X peak) and tokens/s, 1 GPU",
        "value": round(gbps, 1),
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
        "config": {"workload": w.describe() + ("" if groups is None else
                                               f", at most {groups[1]} of {groups[0]} expert groups per token"),
                   "T": T, "H": H, "E": E, "k": k, "R": R,
                   "capacity": C, "shared_expert": w.shared, "kept_rows": N, "tokens_read": T_read,
                   "bytes_per_step": total, "parallelism": "single GPU (R logical destinations)"},
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "per_call_us": {n: round(v * 1e3, 2) for n, v in per_call_ms.items()},
        "timing": "one HIP graph replay per step (four launches)" if graph is not None else "eager launches",
        "ms_per_step_eager": round(ms_eager, 5),
        "per_call_note": "second pass of the same K steps with an event pair around every call",
        "per_call_GBps": {n: round(nbytes[n] / (per_call_ms[n] * 1e-3) / 1e9, 1) for n in nbytes},
        "step_us_spread": spread,
        "step_us_spread_note": "third pass of K steps with one event between consecutive steps",
        "step_us_cold": cold,
        "step_us_cold_note": ("fourth pass of K steps, each after a read of a 1 GiB scratch buffer "
                              "(outside its event pair) that evicts the 256 MB Infinity Cache"),
        "roofline": roofline,
    }
    next_rows = {}
    if fp8:
        next_rows["fp8_dispatch"] = fp8
    if regroup:
        next_rows["recv_regroup"] = regroup
    if tile_return:
        next_rows["tile_signalled_return"] = tile_return
    if next_rows:
        result["next_rows"] = next_rows
    result["load"] = load
    if ms_pipe is not None:
        result["pipelined_two_streams"] = {
            "us_per_step": round(ms_pipe * 1e3, 1), "GBps": round(total / (ms_pipe * 1e-3) / 1e9, 1),
            "tokens_per_s": round(T / (ms_pipe * 1e-3), 1),
            "speedup_vs_one_step_at_a_time": round(ms_per_step / ms_pipe, 3),
            "outputs_bitwise_equal": pipe_equal,
            "note": "two batches in flight on two streams with their own outputs; `value` is one step at a time"}
    if floor:
        result["synthetic_floor"] = floor
    if copy_probe:
        result["copy_probe"] = copy_probe

    if not args.no_cpu_baseline:
        log("cpu baseline: timing the C oracle on the same host arrays")
        sec, reps = cpu_baseline(w, d, args.cpu_seconds)
        model, affinity = host_cpu()
        result["cpu_baseline"] = {
            "value": round(total / sec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the full {w.name} batch (T={T}), {reps} rep(s), median {sec:.2f}s per pass; "
                      f"single-threaded C oracle on {model}",
            "tokens_per_s": round(T / sec, 1),
            "host": {"cpu_model": model, "affinity_cores": affinity, "threads_used": 1},
        }
        log("cpu baseline", result["cpu_baseline"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
