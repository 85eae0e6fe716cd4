#!/usr/bin/env python3
"""Effective HBM bandwidth of the broadcasting binary-operator path on one
MI355X (gfx950): forward + backward of the MLP bias + GeLU workload
(act[4096,1024] + bias[1024] -> GeLU; backward to act and bias), with the
other workloads reported beside it.

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

The oracle (plain C, CPU) is timed on the same workload on the host cores as a
reported baseline only.
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
MAIN = "mlp_bias_gelu"
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
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "hbm_traffic.fetch_write_counters.txt")

def source_hash():
    import glob
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    # device code, kernel argument blocks and the planner decide the traffic
    for p in sorted(glob.glob(os.path.join(root, "broadcast_autograd_amd", "csrc", "*"))):
        if p.endswith((".hip", ".h")) or p.endswith("zk_plan.cpp"):
            with open(p, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def read_traffic(workload, kernel):
    """Counter-measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each
    scaled by a plain copy of known size), or None when the kernels changed
    since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    cur = source_hash()
    for ln in lines:
        p = ln.split()
        if len(p) == 5 and p[0] == "traffic" and p[1] == workload and p[2] == kernel:
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


def copy_ceiling(torch, nbytes=1 << 30, reps=20):
    """Practical HBM ceiling: a plain 1 GiB device-to-device tensor copy
    (read + write), timed the same way (graph, synchronised)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    g = torch.cuda.CUDAGraph()
    dst.copy_(src)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dst.copy_(src)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, dst, g
    torch.cuda.empty_cache()
    return 2 * nbytes / dt / 1e9


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
    fwd_b = sum(c["bytes"] for c in calls if c["kind"] == "fwd")
    bwd_b = sum(c["bytes"] for c in calls if c["kind"] == "bwd")
    fwd_us = sum(c["us"] for c in calls if c["kind"] == "fwd")
    bwd_us = sum(c["us"] for c in calls if c["kind"] == "bwd")
    res = dict(
        workload=name, step_bytes=step_bytes, buffer_sets=len(sets),
        set_bytes=fp, steps=K, warmup=W, seconds=secs,
        ms_per_step=secs / K * 1e3,
        step_gbs=step_bytes * K / secs / 1e9,
        fwd_kernel_gbs=fwd_b / (fwd_us * 1e-6) / 1e9 if fwd_us else None,
        bwd_kernel_gbs=bwd_b / (bwd_us * 1e-6) / 1e9 if bwd_us else None,
        fwd_bwd_kernel_gbs=(fwd_b + bwd_b) / ((fwd_us + bwd_us) * 1e-6) / 1e9,
        calls=calls, profile_reps=reps * len(sets), enqueue_s=enq,
        spin_plus_run_s=spin_total)
    for k in ("step_gbs", "fwd_kernel_gbs", "bwd_kernel_gbs", "fwd_bwd_kernel_gbs"):
        if res[k] is not None:
            res[k.replace("gbs", "frac")] = res[k] * 1e9 / PEAK_HBM
    del sets, graphs, chunk
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_baseline(host, target_s=12.0):
    """The oracle on the whole MLP bias + GeLU step, on the host cores."""
    import oracle
    threads = min(os.cpu_count() or 1, 16)
    oracle.set_threads(threads)

    def step():
        oracle.fwd("add", host["act"], host["bias"], epi=oracle.EPI_GELU)
        oracle.bwd("add", host["g"], host["act"], host["bias"], epi=oracle.EPI_GELU)

    step()
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < target_s:
        step()
        n += 1
    dt = (time.perf_counter() - t0) / n
    return threads, n, dt


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=MAIN, choices=ALL)
    ap.add_argument("--others", default="all",
                    help="comma list of other workloads to report, 'all' or 'none'")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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
    ceiling = copy_ceiling(torch)
    log(f"[bench] 1 GiB device copy: {ceiling:.1f} GB/s (read + write)")
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
            f"{gbs(r['bwd_kernel_gbs'])} GB/s")
        per[w] = r

    # dominant kernel of the main step: the largest total kernel time
    best = None
    for c in res["calls"]:
        for k, us in c["kernels_us"].items():
            if best is None or us > best[2]:
                best = (c, k, us)
    c, kname, kus = best
    hbm = c["bytes"] / (kus * 1e-6) / 1e9
    traffic = read_traffic(args.workload, kname)
    roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": PEAK_HBM / 1e9,
            "unit": "GB/s", "frac": round(hbm * 1e9 / PEAK_HBM, 4),
            "traffic": traffic, "kernel": kname, "call": c["name"],
            "bytes_per_launch": c["bytes"], "us_per_launch": round(kus, 3)}

    cpu = None
    if not args.no_cpu:
        log("[bench] oracle on the host cores ...")
        threads, n, dt = cpu_baseline(gen[MAIN](), args.cpu_seconds)
        step_bytes = per[MAIN]["step_bytes"] if MAIN in per else None
        cpu = {"value": round(step_bytes / dt / 1e9, 3) if step_bytes else None,
               "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{n} full mlp_bias_gelu steps (act[4096,1024]: forward add+GeLU "
                         f"and backward to act and bias), {dt * 1e3:.1f} ms each"}

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
        "config": {"workload": f"{args.workload}: y = GeLU(act[4096,1024] + bias[1024]), "
                               "forward + backward (grad_act, grad_bias)"
                   if args.workload == MAIN else args.workload,
                   "step_bytes": res["step_bytes"],
                   "hbm_peak_frac": round(res["step_frac"], 4),
                   "fwd_kernel_gbs": round(res["fwd_kernel_gbs"], 1),
                   "bwd_kernel_gbs": round(res["bwd_kernel_gbs"], 1),
                   "buffer_sets": res["buffer_sets"],
                   "launch": "hip graphs (one per rotation of buffer sets)",
                   "copy_ceiling_gbs": round(ceiling, 1)},
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
