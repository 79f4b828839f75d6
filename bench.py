#!/usr/bin/env python3
"""Benchmark of the collective datapath on one MI355X.

One step = the bandwidth-sweep workload: R = 8 rank buffers of bf16 N(0,1) at
1, 4, 16, 64 and 256 MiB per rank, each size run as All-Reduce, then
Reduce-Scatter into 8 contiguous chunks, then All-Gather of those chunks;
plus the same three at fp32, 64 MiB.  Inputs are resident in HBM before the
timed region.  ``value`` = algorithmic bytes of the whole step (every input
byte read once, every output byte written once) / step time.

Also reported on the same line:
* ``roofline``: the dominant kernel (the 256 MiB All-Reduce, named as the
  library reports its launch): algorithmic bytes per launch / its mean
  duration from HIP events on the launch stream, recorded around it in the
  timed steps (the only events there), against the 8 TB/s HBM peak;
  ``serial_bound`` sets it against the fastest Reduce-Scatter and
  All-Gather of the same run;
* ``sweep``: per size and collective, the in-step (warm) rate from the same
  number of steps run again after the timed region with events around every
  collective, and a cold rate (a 1 GiB scratch read before each call empties
  the caches);
* ``decode``: the batch-1 decode All-Reduce (8 ranks x 4096 bf16), kernel
  time from events and back-to-back time per call, next to an empty kernel;
* ``seven``: the seven layout-named collectives at 8 x 16 MiB bf16 (us per
  launch replayed from a HIP graph, GB/s, fraction of peak);
* ``chain``: the decode chain, 64 back-to-back All-Reduces per call for every
  b x h payload (b = 1..64, h = 4096, 8192) and every orchestration variant,
  us per All-Reduce, and the mis-speculation rates (speculative waits for
  the flags first above 128 KiB per rank; speculative_always speculates at
  every size);
* ``moe``: MoE dispatch and combine, 4096 x 7168 bf16, 256 experts over 8
  ranks, top-8 (host-built and device-routed maps);
* ``cpu_baseline``: the CPU oracle on a bounded sample of the sweep workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs LIST]
       python bench.py --workload chain|moe|seven   (detailed single workloads)
"""

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "achieved HBM GB/s (% of peak) for 8-rank reduce/copy; µs per batch-1 All-Reduce"
PEAK_GBS = 8000.0
R = 8
SIZES_MIB = [1, 4, 16, 64, 256]
FP32_MIB = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-iters", type=int, default=2000)
    ap.add_argument("--workload", default="sweep", choices=["sweep", "chain", "moe", "seven"],
                    help="sweep (default) is the headline line; the others print "
                         "their own detailed line for the decode chain, MoE and the seven "
                         "collectives")
    ap.add_argument("--legs", default="decode,seven,chain,moe",
                    help="legs measured after the sweep's timed region and added to its line "
                         "(comma list of decode, seven, chain, moe; 'none' for the sweep alone)")
    return ap.parse_args()


def alg_bytes(S_bytes):
    """(AR, RS, AG) algorithmic bytes for S bytes per rank (full tensor)."""
    return 2 * R * S_bytes, (R + 1) * S_bytes, (R + 1) * S_bytes


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the R ranks are buffers in one GPU's HBM; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import reduce_rank_buffers_amd as rrb
    from reduce_rank_buffers_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    rrb.lib()  # loud failure if the library is missing
    if args.workload != "sweep":
        {"chain": bench_chain, "moe": bench_moe, "seven": bench_seven}[args.workload](args, dev)
        return

    # ---- resident inputs and outputs --------------------------------------
    cases = []  # (label, dtype, S_bytes, ins, ar_out, rs_out, ag_out)
    host_inputs = {}  # kept for the CPU oracle leg
    t0 = time.perf_counter()
    for S in SIZES_MIB + ["fp32"]:
        dtype = "f32" if S == "fp32" else "bf16"
        smib = FP32_MIB if S == "fp32" else S
        host = inputs.sweep(smib, dtype=dtype)
        tdt = torch.float32 if dtype == "f32" else torch.int16
        ins = [torch.from_numpy(h.view(np.int16) if dtype == "bf16" else h).to(dev) for h in host]
        if not args.no_cpu_baseline:
            host_inputs[(smib, dtype)] = host
        del host
        n = ins[0].numel()
        ar = [torch.empty(n, dtype=tdt, device=dev) for _ in range(R)]
        rs = [torch.empty(n // R, dtype=tdt, device=dev) for _ in range(R)]
        ag = [torch.empty(n, dtype=tdt, device=dev) for _ in range(R)]
        cases.append((f"{smib}MiB-{dtype}", dtype, smib << 20, ins, ar, rs, ag))
    torch.cuda.synchronize()
    log(f"inputs resident ({time.perf_counter() - t0:.1f} s)")

    step_bytes = sum(sum(alg_bytes(c[2])) for c in cases)
    big = next(c for c in cases if c[0] == "256MiB-bf16")

    ev = lambda: torch.cuda.Event(enable_timing=True)
    per_case_events = {c[0]: [] for c in cases}
    # pre-bound launches: plan, pointers and entry point resolved once
    ops = {label: (rrb.bound("all_reduce", ins, ar), rrb.bound("reduce_scatter", ins, rs),
                   rrb.bound("all_gather", rs, ag))
           for label, dtype, Sb, ins, ar, rs, ag in cases}

    roof_events = []

    def step(record):
        # record = "roof": events around the roofline kernel only (the timed
        # steps); record = "all": events around every collective (the
        # breakdown steps after the timed region).
        for label, *_ in cases:
            op_ar, op_rs, op_ag = ops[label]
            roof = record == "roof" and label == big[0]
            if record == "all" or roof:
                e = [ev() for _ in range(4)]
                e[0].record()
            op_ar()
            if roof:
                e[1].record()
                roof_events.append(e[:2])
            if record == "all":
                e[1].record()
            op_rs()
            if record == "all":
                e[2].record()
            op_ag()
            if record == "all":
                e[3].record()
                per_case_events[label].append(e)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step("roof")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (wall / args.steps) / 1e9
    # Per-collective breakdown: the same number of steps again, with events
    # around every collective (outside the timed region: the 24 event
    # records per step cost about 3% of its time).
    for _ in range(args.steps):
        step("all")
    torch.cuda.synchronize()

    sweep = {}
    for label, dtype, Sb, *_ in cases:
        ab = alg_bytes(Sb)
        times = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)]
                          for e in per_case_events[label]])  # ms
        mean = times.mean(axis=0)
        sweep[label] = {
            k: {"us": round(float(m) * 1e3, 2), "GBps": round(b / (m * 1e-3) / 1e9, 1),
                "frac": round(b / (m * 1e-3) / 1e9 / PEAK_GBS, 4)}
            for k, m, b in zip(("all_reduce", "reduce_scatter", "all_gather"), mean, ab)
        }
        sweep[label]["cache_note"] = "fits in the 256 MB Infinity Cache" if Sb * R * 2 <= (256 << 20) else "above the Infinity Cache"
    ar_bytes = alg_bytes(big[2])[0]
    ar_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in roof_events]))
    achieved = ar_bytes / (ar_ms * 1e-3) / 1e9

    # ---- cold-cache timings (outside the timed region) ---------------------
    # Before each timed call an untimed read of a 1 GiB scratch buffer (written
    # once) evicts the 256 MB Infinity Cache and the L2s and leaves them
    # holding clean lines, so inputs come from HBM and no earlier dirty data
    # is written back during the call; median of 5 per operation.
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    for label, dtype, Sb, *_ in cases:
        ab = alg_bytes(Sb)
        cold = {}
        for k, op, b in zip(("all_reduce", "reduce_scatter", "all_gather"), ops[label], ab):
            ts = []
            for _ in range(5):
                scratch.sum()
                e0, e1 = ev(), ev()
                e0.record()
                op()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            m = float(np.median(ts))
            cold[k] = {"us": round(m * 1e3, 2), "GBps": round(b / (m * 1e-3) / 1e9, 1)}
        sweep[label]["cold"] = cold
    del scratch

    roof_kernel = ops[big[0]][0].kernels()
    # the sweep's buffers are not needed by the legs that follow
    del ops, cases, big
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    legs = [x for x in args.legs.split(",") if x and x != "none"]
    decode = decode_leg(args, torch, rrb, inputs, dev) if "decode" in legs else None

    # ---- copy calibration: a plain 192 MiB copy through the library -------
    # (one rank, SHARD -> SHARD): the known-size kernel that scales the HBM
    # traffic counters, and the practical streaming ceiling next to peak.
    cal_bytes = 192 << 20
    cal_in = torch.empty(cal_bytes // 2, dtype=torch.int16, device=dev).fill_(7)
    cal_out = torch.empty_like(cal_in)
    cal_plan = rrb.Plan(1, cal_bytes // 2, "bf16", rrb.SHARD, rrb.SHARD, "copy")
    for _ in range(3):
        cal_plan.run([cal_in], [cal_out])
    cal_ev = _per_launch_us(torch, lambda: cal_plan.run([cal_in], [cal_out]), 10)
    copy_cal = {"bytes": 2 * cal_bytes, "us": round(float(np.median(cal_ev)), 2),
                "GBps": round(2 * cal_bytes / (float(np.median(cal_ev)) * 1e-6) / 1e9, 1)}
    del cal_in, cal_out

    seven = seven_leg(args, torch, rrb, inputs, dev) if "seven" in legs else None
    moe = moe_leg(args, torch, rrb, inputs, dev) if "moe" in legs else None
    chain = chain_leg(args, torch, rrb, inputs, dev) if "chain" in legs else None
    log(f"legs done: {','.join(legs) or 'none'}")

    # ---- CPU oracle on a bounded sample ------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host_inputs)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16 (one fp32 leg at 64 MiB)",
        "data": "synthetic",
        "config": {
            "workload": "bandwidth sweep: 8 rank buffers x {1,4,16,64,256} MiB bf16 N(0,1), "
                        "All-Reduce -> Reduce-Scatter (8 contiguous chunks) -> All-Gather of "
                        "those chunks, plus fp32 at 64 MiB",
            "ranks": R,
            "step_algorithmic_bytes": step_bytes,
            "parallelism": "single GPU (ranks are HBM buffers)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": roof_kernel,
            "achieved": round(achieved, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic_bytes(),
            "alg_bytes_per_launch": ar_bytes,
            "mean_launch_us": round(ar_ms * 1e3, 2),
            "serial_bound": serial_bound(sweep, ar_ms * 1e3),
        },
        "sweep": sweep,
        "decode": decode,
        "copy_calibration": copy_cal,
        "cpu_baseline": cpu,
        # compact summaries last, so the end of the line carries them
        "seven": seven,
        "moe": moe,
        "chain": chain,
    }
    print(json.dumps(out), flush=True)


def serial_bound(sweep, ar_us):
    """The 256 MiB All-Reduce against this run's own serial read + write
    bound.  An HBM channel's read and write time add up, so with t = bytes
    read / read rate + bytes written / write rate, a Reduce-Scatter (reads
    R*S, writes S) and an All-Gather (reads S, writes R*S) together read and
    write (R+1)*S each, and the All-Reduce (2*R*S: R*S each way) is bounded
    below by (t_RS + t_AG) * R / (R + 1).  t_RS and t_AG are the fastest times
    the run measured for them (in the step or cold), so the bound is the
    tightest this run supports."""
    c = sweep.get("256MiB-bf16")
    if not c or "cold" not in c:
        return None
    t_rs = min(c["reduce_scatter"]["us"], c["cold"]["reduce_scatter"]["us"])
    t_ag = min(c["all_gather"]["us"], c["cold"]["all_gather"]["us"])
    bound = (t_rs + t_ag) * R / (R + 1)
    t_ar = min(ar_us, c["cold"]["all_reduce"]["us"])
    return {"model": "fastest Reduce-Scatter + fastest All-Gather of the same run (in-step or "
                     "cold), times R/(R+1)",
            "rs_us": t_rs, "ag_us": t_ag, "bound_us": round(bound, 2),
            "all_reduce_us": round(t_ar, 2), "frac_of_bound": round(bound / t_ar, 4),
            "bound_frac_of_peak": round(2 * R * (256 << 20) / (bound * 1e-6) / 1e9 / PEAK_GBS, 4)}


def _per_launch_us(torch, fn, iters):
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in ev])


def _back_to_back_us(torch, fn, iters):
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(iters):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t) * 1e6 / iters


def decode_leg(args, torch, rrb, inputs, dev):
    """The batch-1 decode All-Reduce (8 ranks x 4096 bf16) next to an empty
    kernel: events around single host calls, host-issued back to back, and
    replayed from a HIP graph."""
    dec_host = inputs.decode_allreduce()
    dins = [torch.from_numpy(h.view(np.int16)).to(dev) for h in dec_host]
    douts = [torch.empty(4096, dtype=torch.int16, device=dev) for _ in range(R)]
    dec_op = rrb.bound("all_reduce", dins, douts)
    for _ in range(50):
        dec_op()
        rrb.empty_kernel()
    torch.cuda.synchronize()
    it = args.decode_iters
    ar_ev = _per_launch_us(torch, dec_op, it)
    em_ev = _per_launch_us(torch, rrb.empty_kernel, it)
    g_ar = graph_us_per_launch(torch, dec_op)
    g_em = graph_us_per_launch(torch, rrb.empty_kernel)
    return {
        "workload": "All-Reduce, 8 ranks x 4096 bf16 (TP=8 batch-1 decode, hidden 4096)",
        "kernel": dec_op.kernels(),
        "allreduce_graph_us": round(g_ar, 3),
        "empty_kernel_graph_us": round(g_em, 3),
        "graph_note": "64 launches captured in one HIP graph, replayed; us per launch",
        "event_note": "event_us: events around one isolated host call (host launch latency "
                      "included); back_to_back_us: host-issued calls in a loop; the kernel "
                      "durations are in the rocprofv3 kernel trace",
        "allreduce_event_us_p50": round(float(np.median(ar_ev)), 2),
        "allreduce_event_us_p10": round(float(np.percentile(ar_ev, 10)), 2),
        "allreduce_event_us_p90": round(float(np.percentile(ar_ev, 90)), 2),
        "empty_kernel_event_us_p50": round(float(np.median(em_ev)), 2),
        "allreduce_back_to_back_us": round(_back_to_back_us(torch, dec_op, it), 2),
        "empty_back_to_back_us": round(_back_to_back_us(torch, rrb.empty_kernel, it), 2),
    }


SEVEN = ("all_reduce", "reduce_scatter", "all_gather", "all_to_all", "broadcast", "reduce", "gather")


def seven_cases(torch, rrb, inputs, dev):
    """The seven collectives at 8 x 16 MiB bf16, pre-bound: name -> (launch,
    algorithmic bytes).  Roots: Broadcast 3, Reduce 0, Gather 5."""
    S = 16 << 20
    n = S // 2
    c = n // R
    full = [torch.from_numpy(x.view(np.int16)).to(dev) for x in inputs.sweep(16)]
    shards = [x[:c].clone() for x in full]
    outs = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(R)]
    souts = [torch.empty(c, dtype=torch.int16, device=dev) for _ in range(R)]
    return {
        "all_reduce": (rrb.bound("all_reduce", full, outs), 2 * R * S),
        "all_reduce_tree_order": (rrb.bound("all_reduce", full, outs, order="tree"), 2 * R * S),
        "reduce_scatter": (rrb.bound("reduce_scatter", full, souts), (R + 1) * S),
        "all_gather": (rrb.bound("all_gather", shards, outs), (R + 1) * S),
        "all_to_all": (rrb.bound("all_to_all", full, outs), 2 * R * S),
        "broadcast": (rrb.bound("broadcast", full, outs, 3), (R + 1) * S),
        "reduce": (rrb.bound("reduce", full, outs, 0), (R + 1) * S),
        "gather": (rrb.bound("gather", shards, outs, 5), 2 * S),
    }


def _graph_replay_ms(torch, fn, G, reps):
    """fn captured G times in one HIP graph, replayed `reps` times; median ms
    per launch (the graph is released before returning)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(G):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ms = float(np.median(_events_ms(torch, g.replay, reps))) / G
    torch.cuda.synchronize()
    del g
    return ms


def seven_leg(args, torch, rrb, inputs, dev):
    """Compact seven-collective figures: [us per launch replayed from a HIP
    graph, GB/s, fraction of 8 TB/s]."""
    cases = seven_cases(torch, rrb, inputs, dev)
    res = {"workload": "8 ranks x 16 MiB bf16 N(0,1); Broadcast root 3, Reduce root 0, Gather root 5; "
                       "[us per launch (20 launches per HIP graph, replayed), GB/s, frac of 8 TB/s]; "
                       "cache-resident sizes"}
    for name, (fn, b) in cases.items():
        for _ in range(3):
            fn()
        ms = _graph_replay_ms(torch, fn, 20, 10)
        res[name] = [round(ms * 1e3, 2), round(b / (ms * 1e-3) / 1e9, 1),
                     round(b / (ms * 1e-3) / 1e9 / PEAK_GBS, 3)]
    return res


CHAIN_VARIANTS = ("barrier", "dual", "speculative", "speculative_always", "twoshot", "lamport", "graph")


def chain_leg(args, torch, rrb, inputs, dev, reps=10):
    """The decode chain: for every b x h payload, us per All-Reduce of a
    64-deep chain (median call time / 64) for every variant, and the
    mis-speculation rates (failed validations per validation: epochs x ranks
    x slices) of the speculative variant, which waits for the flags first
    above 128 KiB per rank, and of speculative_always, which speculates at
    every size."""
    E = 64
    res = {"workload": "64 back-to-back All-Reduces per call, 8 ranks, b x h bf16 N(0,0.02); "
                       "us per All-Reduce; speculative waits for the flags first above 128 KiB per rank, "
                       "speculative_always speculates at every size",
           "cols": list(CHAIN_VARIANTS) + ["spec_misspec_rate", "spec_always_misspec_rate"]}
    # the memory-model build (RRB_FENCED=1) has no flag-in-data chain: null
    fenced = bool(rrb.lib().rrb_snac_fenced())
    res["ordering"] = "fenced" if fenced else "fence-free"
    for h in (4096, 8192):
        for b in (1, 2, 4, 8, 16, 32, 64):
            n = b * h
            inp = torch.from_numpy(inputs.chain(E, R, n).view(np.int16)).to(dev)
            out = torch.empty_like(inp)
            row = []
            rates = {}
            for v in CHAIN_VARIANTS:
                if fenced and v == "lamport":
                    row.append(None)
                    continue
                ch = rrb.SnacChain(R, n, "bf16", v)
                stats = torch.zeros(4, dtype=torch.int64, device=dev)
                call = ch.bound(inp, out, stats)
                for _ in range(3):
                    call()
                torch.cuda.synchronize()
                stats.zero_()
                ms = float(np.median(_events_ms(torch, call, reps)))
                ch.check()
                row.append(round(ms * 1e3 / E, 3))
                if v.startswith("speculative"):
                    st = stats.cpu().tolist()
                    rates[v] = round(st[0] / max(1, st[3]), 3)  # st[3]: epochs x ranks x slices
                del call
                ch.close()
                # every variant's workspace from the same freed block where the
                # sizes allow, so placement does not differ between variants
                del ch
            res[f"b{b}h{h}"] = row + [rates["speculative"], rates["speculative_always"]]
            del inp, out
    return res


def moe_leg(args, torch, rrb, inputs, dev, reps=20):
    """MoE dispatch / combine at 4096 x 7168 bf16, 256 experts over 8 ranks,
    top-8: [us (median of events around each call), GB/s, frac of 8 TB/s] for
    host-built maps and for device-routed maps into one arena, and the
    device routing time."""
    T, h, E, k = 4096, 7168, 256, 8
    idx, w = inputs.moe_routing(T, E, k)
    shards = inputs.moe_tokens(T, h, R)
    xs = [torch.from_numpy(x.reshape(-1).view(np.int16)).to(dev) for x in shards]
    disp = rrb.MoePlan(R, h, E, idx, w, "dispatch")
    comb = rrb.MoePlan(R, h, E, idx, w, "combine")
    recv = [torch.empty(r * h, dtype=torch.int16, device=dev) for r in disp.rows_per_rank]
    y = [torch.empty(T // R * h, dtype=torch.int16, device=dev) for _ in range(R)]
    d_bytes = T * h * 2 * (1 + k)
    c_bytes = T * h * 2 * (k + 1) + T * k * 8

    def rate(ms, b):
        return [round(ms * 1e3, 2), round(b / (ms * 1e-3) / 1e9, 1), round(b / (ms * 1e-3) / 1e9 / PEAK_GBS, 3)]

    for _ in range(3):
        disp.run(xs, recv)
        comb.run(recv, y)
    d_ms = float(np.median(_events_ms(torch, lambda: disp.run(xs, recv), reps)))
    c_ms = float(np.median(_events_ms(torch, lambda: comb.run(recv, y), reps)))
    ddisp = rrb.MoeDevicePlan(R, T, h, E, k, "dispatch")
    dcomb = rrb.MoeDevicePlan(R, T, h, E, k, "combine", share=ddisp)
    d_idx = torch.from_numpy(idx).to(dev)
    d_w = torch.from_numpy(w).to(dev)
    arena = torch.empty(T * k * h, dtype=torch.int16, device=dev)
    none = [None] * (R - 1)
    for _ in range(3):
        ddisp.route(d_idx, d_w)
        ddisp.run(xs, [arena] + none)
        dcomb.run([arena] + none, y)
    ddisp.check()
    r_ms = float(np.median(_events_ms(torch, lambda: ddisp.route(d_idx, d_w), reps)))
    dd_ms = float(np.median(_events_ms(torch, lambda: ddisp.run(xs, [arena] + none), reps)))
    dc_ms = float(np.median(_events_ms(torch, lambda: dcomb.run([arena] + none, y), reps)))
    return {"workload": "4096 tokens x 7168 bf16, 256 experts over 8 ranks, top-8; [us, GB/s, frac]",
            "dispatch": rate(d_ms, d_bytes), "combine": rate(c_ms, c_bytes),
            "dispatch_arena": rate(dd_ms, d_bytes), "combine_arena": rate(dc_ms, c_bytes),
            "route_us": round(r_ms * 1e3, 2)}


def graph_us_per_launch(torch, fn, per_graph=64, replays=50):
    """Capture `per_graph` back-to-back launches of fn in one HIP graph (on a
    side stream, as torch requires), replay it, and return us per launch."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (replays * per_graph)


def _cold_ms(torch, fn, scratch, reps=5):
    """Median of `reps` calls, each after an untimed read of a 1 GiB scratch
    buffer that evicts the 256 MB Infinity Cache and the L2s (the inputs then
    come from HBM and no earlier dirty data is written back during the call)."""
    ts = []
    for _ in range(reps):
        scratch.sum()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def _events_ms(torch, fn, iters):
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def bench_chain(args, dev):
    """Decode chain: 64 back-to-back All-Reduces (32 layers x 2) per call, for
    each payload b x h and variant; reports us per All-Reduce (kernel time /
    64) next to 64 separate Atom All-Reduce launches."""
    import torch
    import reduce_rank_buffers_amd as rrb
    from reduce_rank_buffers_amd import inputs
    E = 64
    rows = []
    for h in (4096, 8192):
        for b in (1, 2, 4, 8, 16, 32, 64):
            n = b * h
            inp = torch.from_numpy(inputs.chain(E, R, n).view(np.int16)).to(dev)
            out = torch.empty_like(inp)
            res = {"b": b, "h": h, "payload_bytes": n * 2}
            for v in CHAIN_VARIANTS:
                if v == "lamport" and rrb.lib().rrb_snac_fenced():
                    continue  # the memory-model build has no flag-in-data chain
                ch = rrb.SnacChain(R, n, "bf16", v)
                stats = torch.zeros(4, dtype=torch.int64, device=dev)
                call = ch.bound(inp, out, stats)  # marshalled once
                for _ in range(3):
                    call()
                stats.zero_()
                ms = _events_ms(torch, call, max(5, args.steps))
                ch.check()
                st = stats.cpu().tolist()
                res[v] = {"us_per_allreduce": round(float(np.median(ms)) * 1e3 / E, 3),
                          "misspec_per_call": round(st[0] / max(5, args.steps), 2),
                          "retries_per_call": round(st[1] / max(5, args.steps), 2),
                          "misspec_rate": round(st[0] / max(1, st[3]), 3)}
                del call
                ch.close()  # HIP objects released here, not at interpreter exit
                del ch  # its workspace is free before the next variant allocates
            ops = [rrb.bound("all_reduce", [inp[e, r] for r in range(R)],
                             [out[e, r] for r in range(R)]) for e in range(E)]

            def separate():
                for op in ops:
                    op()
            for _ in range(3):
                separate()
            ms = _events_ms(torch, separate, max(5, args.steps))
            res["separate_launches"] = {"us_per_allreduce": round(float(np.median(ms)) * 1e3 / E, 3)}
            res["separate_launches_graph"] = {
                "us_per_allreduce": round(graph_us_per_launch(torch, separate, per_graph=1, replays=20) / E, 3)}
            rows.append(res)
            log(json.dumps(res))
    # Chains of every layout-named collective through the plan-driven SNAC
    # kernel: 8 ranks, a 16 KiB bf16 tensor per rank (shards of 2 KiB).
    n = 8192
    plan_rows = {}
    for name in ("all_reduce", "reduce_scatter", "all_gather", "all_to_all", "broadcast",
                 "reduce", "gather"):
        lin, lout, op = {
            "all_reduce": (rrb.PARTIAL, rrb.REPLICATED, "reduce"),
            "reduce_scatter": (rrb.PARTIAL, rrb.SHARD, "reduce"),
            "all_gather": (rrb.SHARD, rrb.REPLICATED, "copy"),
            "all_to_all": (rrb.BLOCK_ROW, rrb.BLOCK_COL, "copy"),
            "broadcast": (rrb.ROOT(3), rrb.REPLICATED, "copy"),
            "reduce": (rrb.PARTIAL, rrb.ROOT(0), "reduce"),
            "gather": (rrb.SHARD, rrb.ROOT(5), "copy"),
        }[name]
        plan = rrb.Plan(R, n, "bf16", lin, lout, op)
        res = {}
        for v in ("barrier", "dual", "speculative", "graph"):
            ch = rrb.SnacPlanChain(plan, v)
            si, so = ch.strides
            pin = torch.from_numpy(inputs.chain(E, R, si, kind=40).view(np.int16)).to(dev)
            pout = torch.empty((E, R, so), dtype=torch.int16, device=dev)
            stats = torch.zeros(4, dtype=torch.int64, device=dev)
            call = ch.bound(pin, pout, stats)
            for _ in range(3):
                call()
            stats.zero_()
            ms = _events_ms(torch, call, max(5, args.steps))
            ch.check()
            res[v] = {"us_per_collective": round(float(np.median(ms)) * 1e3 / E, 3),
                      "misspec_per_call": round(stats[0].item() / max(5, args.steps), 2)}
            del call
            ch.close()
            del ch, pin, pout  # freed before the next variant allocates
        plan_rows[name] = res
        log(json.dumps({name: res}))
    print(json.dumps({"metric": "us per All-Reduce in a 64-deep decode chain", "unit": "us",
                      "higher_is_better": False, "workload": "decode chain, 8 ranks, b x h bf16 N(0,0.02)",
                      "rows": rows,
                      "plan_chains": {"workload": "64-deep chains of each layout-named collective, "
                                                  "8 ranks, 16 KiB bf16 tensor per rank",
                                      "rows": plan_rows}}), flush=True)


def bench_moe(args, dev):
    """MoE dispatch / combine: 4096 tokens x 7168 bf16, 256 experts over 8
    ranks, top-8."""
    import torch
    import reduce_rank_buffers_amd as rrb
    from reduce_rank_buffers_amd import inputs
    T, h, E, k = 4096, 7168, 256, 8
    idx, w = inputs.moe_routing(T, E, k)
    shards = inputs.moe_tokens(T, h, R)
    xs = [torch.from_numpy(s.reshape(-1).view(np.int16)).to(dev) for s in shards]
    disp = rrb.MoePlan(R, h, E, idx, w, "dispatch")
    comb = rrb.MoePlan(R, h, E, idx, w, "combine")
    recv = [torch.empty(r * h, dtype=torch.int16, device=dev) for r in disp.rows_per_rank]
    y = [torch.empty(T // R * h, dtype=torch.int16, device=dev) for _ in range(R)]
    for _ in range(3):
        disp.run(xs, recv)
        comb.run(recv, y)
    d_ms = float(np.median(_events_ms(torch, lambda: disp.run(xs, recv), max(10, args.steps))))
    c_ms = float(np.median(_events_ms(torch, lambda: comb.run(recv, y), max(10, args.steps))))
    d_bytes = T * h * 2 * (1 + k)
    c_bytes = T * h * 2 * (k + 1) + T * k * 8
    # device-side routing maps (no host round trip per step) into one arena
    ddisp = rrb.MoeDevicePlan(R, T, h, E, k, "dispatch")
    dcomb = rrb.MoeDevicePlan(R, T, h, E, k, "combine", share=ddisp)
    d_idx = torch.from_numpy(idx).to(dev)
    d_w = torch.from_numpy(w).to(dev)
    arena = torch.empty(T * k * h, dtype=torch.int16, device=dev)
    none = [None] * (R - 1)
    for _ in range(3):
        ddisp.route(d_idx, d_w)
        ddisp.run(xs, [arena] + none)
        dcomb.run([arena] + none, y)
    r_ms = float(np.median(_events_ms(torch, lambda: ddisp.route(d_idx, d_w), max(10, args.steps))))
    dd_ms = float(np.median(_events_ms(torch, lambda: ddisp.run(xs, [arena] + none), max(10, args.steps))))
    dc_ms = float(np.median(_events_ms(torch, lambda: dcomb.run([arena] + none, y), max(10, args.steps))))
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    cd_ms = _cold_ms(torch, lambda: ddisp.run(xs, [arena] + none), scratch)
    cc_ms = _cold_ms(torch, lambda: dcomb.run([arena] + none, y), scratch)
    del scratch
    t0 = time.perf_counter()
    for _ in range(10):
        rrb.MoePlan(R, h, E, idx, w, "dispatch")
    host_plan_ms = (time.perf_counter() - t0) * 1e3 / 10
    print(json.dumps({"metric": "achieved HBM GB/s, MoE dispatch / combine", "unit": "GB/s",
                      "workload": "MoE 4096 tokens x 7168 bf16, 256 experts over 8 ranks, top-8",
                      "dispatch": {"us": round(d_ms * 1e3, 2), "GBps": round(d_bytes / (d_ms * 1e-3) / 1e9, 1),
                                   "frac": round(d_bytes / (d_ms * 1e-3) / 1e9 / PEAK_GBS, 4), "bytes": d_bytes},
                      "combine": {"us": round(c_ms * 1e3, 2), "GBps": round(c_bytes / (c_ms * 1e-3) / 1e9, 1),
                                  "frac": round(c_bytes / (c_ms * 1e-3) / 1e9 / PEAK_GBS, 4), "bytes": c_bytes},
                      "rows_per_rank": disp.rows_per_rank,
                      "device_routing": {
                          "route_us": round(r_ms * 1e3, 2),
                          "host_plan_build_and_upload_ms": round(host_plan_ms, 2),
                          "dispatch_arena": {"us": round(dd_ms * 1e3, 2),
                                             "GBps": round(d_bytes / (dd_ms * 1e-3) / 1e9, 1)},
                          "combine_arena": {"us": round(dc_ms * 1e3, 2),
                                            "GBps": round(c_bytes / (dc_ms * 1e-3) / 1e9, 1)},
                          "cold": {"note": "one call after a 1 GiB cache-evicting read, median of 5",
                                   "dispatch_arena_us": round(cd_ms * 1e3, 2),
                                   "dispatch_arena_GBps": round(d_bytes / (cd_ms * 1e-3) / 1e9, 1),
                                   "combine_arena_us": round(cc_ms * 1e3, 2),
                                   "combine_arena_GBps": round(c_bytes / (cc_ms * 1e-3) / 1e9, 1)}}}),
          flush=True)


def bench_seven(args, dev):
    """The seven layout-named collectives at 16 MiB bf16 per rank."""
    import torch
    import reduce_rank_buffers_amd as rrb
    from reduce_rank_buffers_amd import inputs
    cases = seven_cases(torch, rrb, inputs, dev)
    # Two timings per collective: G launches captured in one HIP graph and
    # replayed (us per launch, no host gaps: the GB/s figure), and events
    # around one host-issued launch (event_us, host launch gaps included).
    G = 20
    res = {}
    for name, (fn, b) in cases.items():
        for _ in range(3):
            fn()
        ev_ms = float(np.median(_events_ms(torch, fn, max(10, args.steps))))
        ms = _graph_replay_ms(torch, fn, G, max(10, args.steps))
        res[name] = {"us": round(ms * 1e3, 2), "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                     "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_GBS, 4), "bytes": b,
                     "event_us": round(ev_ms * 1e3, 2)}
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    for name, (fn, b) in cases.items():
        cm = _cold_ms(torch, fn, scratch)
        res[name]["cold_event_us"] = round(cm * 1e3, 2)
        res[name]["cold_GBps"] = round(b / (cm * 1e-3) / 1e9, 1)
    del scratch
    print(json.dumps({"metric": "achieved GB/s, seven collectives, 8 ranks x 16 MiB bf16 (cache-resident sizes)",
                      "unit": "GB/s", "timing": f"{G} launches in one HIP graph, replayed; us per launch; "
                                                "cold_event_us: one host-issued launch after a 1 GiB "
                                                "cache-evicting read, median of 5",
                      "results": res}), flush=True)


def kernel_source_digest():
    """sha256 over the sources that define the Atom kernels."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "reduce_rank_buffers_amd", "csrc")
    for f in ("rrb_atom.hip", "rrb_kernels.h"):
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes():
    """Counter-measured HBM bytes per launch of the roofline kernel, from the
    committed rocprofv3 --pmc summary -- or None if the kernel sources changed
    since those counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "hbm_traffic_allreduce_256mib.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(host_inputs):
    """The oracle, untuned, on one whole step of the same workload: All-Reduce
    -> Reduce-Scatter -> All-Gather at every sweep size (bf16 1..256 MiB and
    fp32 64 MiB per rank), on the same host arrays the GPU received."""
    from oracle import collectives as C
    # Whole steps, repeated until at least 10 s of CPU work (at most 3 steps).
    t0 = time.perf_counter()
    total = 0
    steps = 0
    while steps < 3 and (steps == 0 or time.perf_counter() - t0 < 10.0):
        for (smib, dtype), ins in host_inputs.items():
            C.all_reduce(ins, dtype)
            rs = C.reduce_scatter(ins, dtype)
            C.all_gather(rs)
            total += sum(alg_bytes(smib << 20))
        steps += 1
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    # The same oracle functions on contiguous element ranges in a thread pool
    # (numpy releases the GIL inside its loops).
    from concurrent.futures import ThreadPoolExecutor
    workers = max(1, min(16, cores))

    def ranged(args):
        ins, dtype, a, b = args
        C.all_reduce([x[a:b] for x in ins], dtype)
        rs = C.reduce_scatter([x[a:b] for x in ins], dtype)
        C.all_gather(rs)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as pool:
        jobs = []
        for (smib, dtype), ins in host_inputs.items():
            n = len(ins[0])
            step = -(-n // (workers * R)) * R  # ranges of a multiple of R elements
            jobs += [(ins, dtype, a, min(n, a + step)) for a in range(0, n, step)]
        list(pool.map(ranged, jobs))
    dt_threads = time.perf_counter() - t0
    return {"value": round(total / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "host_cores_visible": cores, "cpu_model": model, "kind": "oracle",
            "seconds": round(dt, 2), "steps": steps,
            "sample": f"{steps} full step(s): All-Reduce -> Reduce-Scatter -> All-Gather, 8 ranks x "
                      "{1,4,16,64,256} MiB bf16 + 64 MiB fp32 (numpy, single thread)",
            "threaded": {"value": round(total / dt_threads / 1e9, 3), "unit": "GB/s",
                         "cores": workers, "seconds": round(dt_threads, 2),
                         "sample": "the same step, the oracle's functions applied to contiguous "
                                   "element ranges in a thread pool"}}


if __name__ == "__main__":
    main()
