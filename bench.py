#!/usr/bin/env python3
"""Effective HBM bandwidth of the broadcasting binary-operator path on one
MI355X (gfx950): forward + backward of the GPT-scale residual workload
(out = h[16,2048,4096] * gamma[4096] + resid[16,2048,4096]; backward to h,
gamma and resid), the largest of the five configurations, with the other
workloads reported beside it.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step = the workload's forward and backward library calls on one batch of
inputs resident in HBM.  Steps rotate over several independent buffer sets so
that no step finds its inputs in the 256 MB last-level cache; each buffer
set's step is captured once in a HIP graph and replayed.  The timed region is
exactly K steps between two device synchronisations.

Per-kernel durations come from HIP events recorded by the library around each
kernel on its own stream (zk_profile_*), with the whole sequence queued behind
a bounded spin kernel so that the host's enqueue time never shows up between
the events.  Algorithmic bytes of a call = 4 x (distinct input elements read
+ elements written).

Each configuration is reported with its forward kernels' and its reducing
backward call's fraction of the 8 TB/s HBM peak, against the targets of 80%
(forward) and 65% (backward reduce-to-shape).

The oracle (plain C, CPU) is timed on a row slice of the same workload on one
host core and on all the cores this process may use, as a reported baseline
only.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s
METRIC = "effective HBM GB/s (fwd, fwd+bwd) and % of MI355X HBM peak per config"
MAIN = "gpt_residual"
# the five configurations (4 has two parts) and their workloads
CONFIGS = {"xy_plus_x": "1", "mlp_bias_gelu": "2", "attn_scale_mask": "3",
           "strided_transposed": "4a", "rank8_div": "4b", "gpt_residual": "5"}
TARGETS = {"fwd": 0.80, "bwd_reduce": 0.65}
MAIN_DESC = ("gpt_residual: out = h[16,2048,4096] * gamma[4096] + resid[16,2048,4096], "
             "forward (mul, add) + backward (grad_h, grad_gamma reduced over 32768 rows, "
             "grad_resid)")
ALL = ["xy_plus_x", "mlp_bias_gelu", "attn_scale_mask", "strided_transposed",
       "rank8_div", "gpt_residual",
       # the three two-operator expressions again, each as one fused call per
       # direction (fewer bytes: the intermediate is never stored)
       "xy_plus_x_fused", "attn_scale_mask_fused", "gpt_residual_fused",
       # the other reductions: mean of the per-token loss and its gradient,
       # ClipGradNorm over the GPT configuration's parameter gradients
       "gpt_loss_mean_clip",
       # per-row statistics: LayerNorm mean / variance, softmax max / sum exp
       "gpt_row_stats",
       # the attention mask's gradient: scores' gradient summed to [1,1,1024,1024]
       "attn_mask_grad"]
ROTATE_BYTES = 1 << 30  # per-workload footprint of the rotating buffer sets
MAX_SETS = 32
# counter summaries whose `traffic` lines give HBM bytes per launch
TRAFFIC_GLOB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "*.fetch_write_counters.txt")

def read_traffic(workload, kernel):
    """Counter-measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each
    scaled by a plain copy of known size), or None when the kernels changed
    since the counters were taken."""
    import glob
    from broadcast_autograd_amd.profsum import source_hash
    cur = None
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        with open(path) as f:
            for ln in f:
                p = ln.split()
                if len(p) == 5 and p[0] == "traffic" and p[1] == workload and p[2] == kernel:
                    cur = cur or source_hash()
                    return int(p[3]) if p[4] == cur else None
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def footprint(wl):
    import torch
    seen, tot = set(), 0
    for v in vars(wl).values():
        if isinstance(v, torch.Tensor) and v.is_cuda:
            p = v.untyped_storage().data_ptr()
            if p not in seen:
                seen.add(p)
                tot += v.untyped_storage().nbytes()
    return tot


def make_sets(name, host):
    """Independent buffer sets of one workload (same values, own memory)."""
    from broadcast_autograd_amd import steps
    cls = steps.WORKLOAD_CLASSES[name]
    first = cls(host=host)
    fp = footprint(first)
    n = int(min(MAX_SETS, max(1, math.ceil(ROTATE_BYTES / max(fp, 1)))))
    return [first] + [cls(host=host) for _ in range(n - 1)], fp


def capture(sets, torch):
    """One HIP graph per buffer set, each holding one whole step."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sets:
            s.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for s in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.run()
        graphs.append(g)
    # all sets' steps back to back in one graph: fewer graph launches
    chunk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(chunk):
        for s in sets:
            s.run()
    torch.cuda.synchronize()
    return graphs, chunk


def outputs(wl, torch):
    names = [k for k, v in vars(wl).items() if isinstance(v, torch.Tensor)
             and (k.startswith(("grad_", "out")) or k in ("t", "z", "y"))]
    return {k: getattr(wl, k).detach().clone() for k in sorted(names)}


def check_graph_replays(sets, graphs, torch):
    """Every replay must reproduce the eager result bit for bit."""
    sets[0].run()
    torch.cuda.synchronize()
    ref = outputs(sets[0], torch)
    for _ in range(3):
        graphs[0].replay()
        torch.cuda.synchronize()
        got = outputs(sets[0], torch)
        for k in ref:
            if not torch.equal(ref[k].view(torch.int32), got[k].view(torch.int32)):
                raise RuntimeError(f"graph replay differs from eager on {k}")
        sets[0].run()  # eager work between replays
        torch.cuda.synchronize()


def run_steps(graphs, chunk, K):
    """Exactly K steps: whole chunks of len(graphs) steps, then single ones."""
    n = len(graphs)
    for _ in range(K // n):
        chunk.replay()
    for k in range(K % n):
        graphs[k].replay()


def time_steps(graphs, chunk, K, W, torch):
    run_steps(graphs, chunk, W)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(graphs, chunk, K)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def calibration(torch, nbytes=1 << 30, reps=20):
    """Practical HBM ceilings: 1 GiB copied device to device (read + write
    counted) by the library's own streaming copy (zk_materialize of a dense
    tensor: 128-bit non-temporal loads and stores) and by hipMemcpyAsync
    (torch's copy_ of a contiguous tensor), each the median of `reps` copies
    timed with events on the stream it runs on."""
    from broadcast_autograd_amd import zk
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    out = {}
    for name, fn in (("zk_copy_16B", lambda: zk.materialize(src, out=dst)),
                     ("hipMemcpyAsync_DtoD", lambda: dst.copy_(src))):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        out[name] = round(2 * nbytes / float(np.median(ts)) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def profile_calls(sets, reps, torch):
    """Per-kernel event durations.  Returns {call index: {kernel: [ms,...]}}."""
    from broadcast_autograd_amd import zk
    wl0 = sets[0]
    ncalls = len(wl0.calls)
    # kernels per call, learned from one profiled step
    zk.profile_start(64)
    torch.cuda.synchronize()
    per_call = []
    for c in wl0.calls:
        zk.profile_stop()
        zk.profile_start(64)
        c()
        torch.cuda.synchronize()
        per_call.append([k for k, _ in zk.profile_read()])
    zk.profile_stop()
    nk = sum(len(x) for x in per_call)
    cap = nk * reps * len(sets) + 16
    zk.profile_start(cap)
    # queue everything behind a bounded spin so enqueue gaps stay outside
    t0 = time.perf_counter()
    torch.cuda._sleep(int(2e8))
    for _ in range(reps):
        for s in sets:
            s.run()
    enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    spin_total = time.perf_counter() - t0
    recs = zk.profile_read(cap)
    zk.profile_stop()
    # per call and kernel name: the summed duration of that kernel's launches
    # in one step (a call may launch one kernel several times)
    out = {i: {} for i in range(ncalls)}
    it = iter(recs)
    for _ in range(reps * len(sets)):
        for i, ks in enumerate(per_call):
            step = {}
            for k in ks:
                name, ms = next(it)
                assert name == k, (name, k)
                step[k] = step.get(k, 0.0) + ms
            for k, ms in step.items():
                out[i].setdefault(k, []).append(ms)
    return out, per_call, enq, spin_total


def spin_seconds(torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(int(2e8))
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def measure(name, host, K, W, torch, reps=None, check=True):
    from broadcast_autograd_amd import steps  # noqa: F401
    sets, fp = make_sets(name, host)
    graphs, chunk = capture(sets, torch)
    if check:
        check_graph_replays(sets, graphs, torch)
    secs = time_steps(graphs, chunk, K, W, torch)
    wl = sets[0]
    step_bytes = wl.step_bytes()
    if reps is None:
        reps = max(1, 64 // len(sets))
    prof, per_call, enq, spin_total = profile_calls(sets, reps, torch)
    calls = []
    for i, c in enumerate(wl.calls):
        kern = {k: float(np.mean(v)) * 1e3 for k, v in prof[i].items()}  # us
        us = sum(kern.values())
        calls.append(dict(name=c.name, kind=c.kind, bytes=c.bytes, elements=c.elements, us=us,
                          kernels_us=kern, gbs=c.bytes / (us * 1e-6) / 1e9 if us else None))
    for cc, c in zip(calls, wl.calls):
        cc["reduce"] = c.reduce
    fwd_b = sum(c["bytes"] for c in calls if c["kind"] == "fwd")
    bwd_b = sum(c["bytes"] for c in calls if c["kind"] == "bwd")
    fwd_us = sum(c["us"] for c in calls if c["kind"] == "fwd")
    bwd_us = sum(c["us"] for c in calls if c["kind"] == "bwd")
    red_b = sum(c["bytes"] for c in calls if c["kind"] == "bwd" and c["reduce"])
    red_us = sum(c["us"] for c in calls if c["kind"] == "bwd" and c["reduce"])
    res = dict(
        workload=name, step_bytes=step_bytes, buffer_sets=len(sets),
        set_bytes=fp, steps=K, warmup=W, seconds=secs,
        ms_per_step=secs / K * 1e3,
        step_gbs=step_bytes * K / secs / 1e9,
        fwd_kernel_gbs=fwd_b / (fwd_us * 1e-6) / 1e9 if fwd_us else None,
        bwd_kernel_gbs=bwd_b / (bwd_us * 1e-6) / 1e9 if bwd_us else None,
        fwd_bwd_kernel_gbs=(fwd_b + bwd_b) / ((fwd_us + bwd_us) * 1e-6) / 1e9,
        bwd_reduce_kernel_gbs=red_b / (red_us * 1e-6) / 1e9 if red_us else None,
        calls=calls, profile_reps=reps * len(sets), enqueue_s=enq,
        spin_plus_run_s=spin_total)
    for k in ("step_gbs", "fwd_kernel_gbs", "bwd_kernel_gbs", "fwd_bwd_kernel_gbs",
              "bwd_reduce_kernel_gbs"):
        if res[k] is not None:
            res[k.replace("gbs", "frac")] = res[k] * 1e9 / PEAK_HBM
    if name in CONFIGS:
        res["config"] = CONFIGS[name]
        res["targets"] = {
            "fwd": {"frac": round(res["fwd_kernel_frac"], 4), "target": TARGETS["fwd"],
                    "met": res["fwd_kernel_frac"] >= TARGETS["fwd"]},
            "bwd_reduce": {"frac": round(res["bwd_reduce_kernel_frac"], 4),
                           "target": TARGETS["bwd_reduce"],
                           "met": res["bwd_reduce_kernel_frac"] >= TARGETS["bwd_reduce"]}}
    del sets, graphs, chunk
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s=10.0, rows=256):
    """The oracle on a row slice of the residual workload (h[1,rows,4096],
    the same per-row work as every one of the full workload's 32768 rows):
    forward mul and add, backward to h, gamma and resid, repeated for about
    target_s seconds, once on one thread and once on every core this
    process may use.  GB/s = the slice step's algorithmic bytes / time."""
    import oracle
    from broadcast_autograd_amd import workloads as Wk
    host = Wk.gpt_residual(1, rows, 4096)
    nh, ng = host["h"].size, host["gamma"].size
    step_bytes = 4 * ((nh + ng + nh) + (3 * nh) + (3 * nh + ng + nh + ng) + (2 * nh))

    def step():
        t = oracle.fwd("mul", host["h"], host["gamma"])
        oracle.fwd("add", t, host["resid"])
        oracle.bwd("mul", host["g"], host["h"], host["gamma"])
        oracle.bwd("add", host["g"], t, host["resid"], want=(False, True))

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    allc = max(1, min(avail, int(omp))) if omp and omp.isdigit() else avail
    res = {}
    for threads in (1, allc):
        oracle.set_threads(threads)
        step()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < target_s:
            step()
            n += 1
        dt = (time.perf_counter() - t0) / n
        res[threads] = (n, dt, step_bytes / dt / 1e9)
    return res, allc, avail, rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=MAIN, choices=ALL)
    ap.add_argument("--others", default="all",
                    help="comma list of other workloads to report, 'all' or 'none'")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--other-steps", type=int, default=None,
                    help="timed steps of each other workload (default 40 for the "
                         "1 GB-scale ones, 400 for the small ones)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharded, each GPU would run the same kernels on 1/N of the rows, "
              "then gather the small reduced gradients).", file=sys.stderr)
        sys.exit(2)
    import torch
    from broadcast_autograd_amd import zk, workloads as Wk
    zk.lib()  # raises if the library is not built
    torch.cuda.set_device(0)
    gen = {"xy_plus_x": Wk.xy_plus_x, "mlp_bias_gelu": Wk.mlp_bias_gelu,
           "attn_scale_mask": Wk.attn_scale_mask,
           "strided_transposed": Wk.strided_transposed, "rank8_div": Wk.rank8,
           "gpt_residual": Wk.gpt_residual}
    for w in ("xy_plus_x", "attn_scale_mask", "gpt_residual"):
        gen[w + "_fused"] = gen[w]
    gen["gpt_loss_mean_clip"] = Wk.gpt_loss_mean_clip
    gen["gpt_row_stats"] = Wk.gpt_row_stats
    gen["attn_mask_grad"] = Wk.attn_mask_grad
    log(f"[bench] device {torch.cuda.get_device_name(0)}; spin check "
        f"{spin_seconds(torch) * 1e3:.1f} ms")
    calib = calibration(torch)
    log(f"[bench] 1 GiB device copies (read + write): {calib}")
    main_host = gen[args.workload]()
    log(f"[bench] main workload {args.workload}: {args.steps} steps")
    res = measure(args.workload, main_host, args.steps, args.warmup, torch)
    log(f"[bench]   {res['ms_per_step'] * 1e3:.2f} us/step, {res['step_gbs']:.1f} GB/s")
    if res["enqueue_s"] > res["spin_plus_run_s"] * 0.8:
        log("[bench]   warning: enqueue time close to spin length; kernel event "
            "times may include host gaps")

    per = {args.workload: {k: v for k, v in res.items() if k != "calls"}}
    per[args.workload]["calls"] = res["calls"]
    others = [] if args.others == "none" else (
        [w for w in ALL if w != args.workload] if args.others == "all"
        else [w for w in args.others.split(",") if w and w != args.workload])
    for w in others:
        big = w.replace("_fused", "") in ("attn_scale_mask", "gpt_residual",
                                          "strided_transposed", "attn_mask_grad")
        K = args.other_steps or (40 if big else 400)
        log(f"[bench] workload {w}: {K} steps")
        r = measure(w, gen[w](), K, K // 10, torch)
        def gbs(v):
            return "-" if v is None else f"{v:.1f}"
        log(f"[bench]   {r['ms_per_step'] * 1e3:.2f} us/step, {r['step_gbs']:.1f} GB/s; "
            f"fwd kernels {gbs(r['fwd_kernel_gbs'])} GB/s, bwd kernels "
            f"{gbs(r['bwd_kernel_gbs'])} GB/s, reducing bwd call "
            f"{gbs(r['bwd_reduce_kernel_gbs'])} GB/s")
        per[w] = r

    # dominant kernel of the main step: the largest total kernel time
    best = None
    for c in res["calls"]:
        for k, us in c["kernels_us"].items():
            if best is None or us > best[2]:
                best = (c, k, us)
    c, kname, kus = best
    # the launch's own algorithmic bytes: a reducing call's stage-1 kernel
    # moves everything but the reduced gradient its stage 2 writes
    kbytes = c["bytes"]
    if c["reduce"] and "red_final" in c["kernels_us"] and kname != "red_final":
        kbytes -= 4 * c["reduce"]
    hbm = kbytes / (kus * 1e-6) / 1e9
    traffic = read_traffic(args.workload, kname)
    roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": PEAK_HBM / 1e9,
            "unit": "GB/s", "frac": round(hbm * 1e9 / PEAK_HBM, 4),
            "traffic": traffic, "kernel": kname, "call": c["name"],
            "bytes_per_launch": kbytes, "us_per_launch": round(kus, 3)}

    cpu = None
    if not args.no_cpu:
        log("[bench] oracle on the host cores ...")
        res_cpu, allc, avail, rows = cpu_baseline(args.cpu_seconds)
        n1, dt1, v1 = res_cpu[1]
        na, dta, va = res_cpu[allc]
        cpu = {"value": round(va, 4), "unit": "GB/s", "cores": allc, "kind": "oracle",
               "sample": f"gpt_residual on h[1,{rows},4096] (a {rows}-row slice of the "
                         f"32768 rows; same per-row work): forward mul and add, backward "
                         f"to h, gamma and resid; {na} steps of {dta * 1e3:.1f} ms on "
                         f"{allc} threads, {n1} steps of {dt1 * 1e3:.1f} ms on 1 thread",
               "one_core": {"value": round(v1, 4), "cores": 1},
               "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
               "cpus_available": avail}

    line = {
        "metric": METRIC,
        "value": round(res["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": MAIN_DESC if args.workload == MAIN else args.workload,
                   "step_bytes": res["step_bytes"],
                   "hbm_peak_frac": round(res["step_frac"], 4),
                   "fwd_kernel_gbs": round(res["fwd_kernel_gbs"], 1),
                   "bwd_kernel_gbs": round(res["bwd_kernel_gbs"], 1),
                   "buffer_sets": res["buffer_sets"],
                   "launch": "hip graphs (one per rotation of buffer sets)",
                   "fwd_frac": round(res["fwd_kernel_frac"], 4),
                   "bwd_reduce_frac": round(res["bwd_reduce_kernel_frac"], 4)
                   if res.get("bwd_reduce_kernel_frac") is not None else None,
                   "calibration_copy_gbs": calib},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_config": {w: {k: (round(v, 4) if isinstance(v, float) else v)
                           for k, v in r.items() if k not in ("calls",)}
                       | {"calls": [{k: (round(v, 3) if isinstance(v, float) else v)
                                     for k, v in cc.items()} for cc in r["calls"]]}
                       for w, r in per.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
