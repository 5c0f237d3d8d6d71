"""Benchmark: MoE-block decode of the channel-selection reader on one MI355X.

One step = one batch-1 decode of the Qwen3-30B-A3B-shaped routed-expert layer
(hidden 2048, 128 experts, intermediate 768, top-8: 6144 candidates) at the
17.8% read budget (k = 756): rotate + select, sketch screen, score + exact
top-k, exact gather of the kept channels, rank-32 recovery.

Method:
  * one layer is built once and cloned into --layers byte-identical copies at
    distinct device addresses; consecutive steps use different copies and
    different tokens, so no step finds its bytes in L2 or the 256 MB
    Infinity Cache (40 copies x ~13.5 MB touched per token >> 256 MB);
  * the steps are captured once in a HIP graph (one graph = one pass over all
    copies) and replayed; HIP events on the replay stream bracket the timed
    replays, after warm-up replays;
  * inputs (x, expert ids, routing weights) are synthetic and already resident
    in device memory when the timed region starts;
  * the per-kernel durations come from each kernel launched alone
    (cfr_reader_decode_stage), back to back over the layer copies in a HIP
    graph timed with events on its replay stream; `roofline` divides the
    dominant kernel's algorithmic bytes by its duration, and `traffic` is the
    HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter
    summary (null when the kernel source changed since it was taken);
  * the dense-BF16 routed-expert block on the same weights and the CPU oracle
    (float64, host cores, bounded sample) are reported beside the reader;
  * a batch-1 layer step per copy (`layer_step_batch1`): the library's
    routing of RMSNorm(x) with the fused pre-norm, then the decode of the
    normed token with its output added to the residual stream x in the
    decode's last kernel; the same with the dense block, and the routing
    alone;
  * the 48-layer stack (`stack_48l`, independent weights per layer): one
    batch-1 step of route + decode + residual per layer as one HIP graph,
    beside the same chain with the dense block (`--stack` times it alone);
  * the 28.7% budget is timed the same way on a second set of layer copies
    built for the ranking the method uses from that budget on (whole sketch,
    expected squared error with rho), k chosen by the read accounting;
  * the Qwen3-235B-A22B-shaped layer (hidden 4096, 128 experts, intermediate
    1536) at batch 8 and k = 1511, on 8 copies, beside its dense block;
  * batch-shared selection (one top-k per call over the call's distinct
    routed experts, k = the per-token budget times distinct experts / top)
    at batch 4 and on the Qwen3-235B-A22B layer at batch 8;
  * the reader over a synthetic 4-bit checkpoint of the batch-1 layer
    (`int4_exact_rows`: exact rows in 4 bits with fp16 group scales, sketch
    unchanged) at k = 756 and at the k reading 18.9% of the BF16 routed
    bytes, beside the 4-bit dense block.

Prints ONE JSON line.  --gpus above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MIN_PASSES = 5      # graph passes per timed figure, at least
MIN_DECODES = 200   # decodes per timed figure, at least
METRIC = "MoE-block µs/token and achieved HBM GB/s at 17.8% reads, batch 1"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--layers", type=int, default=40, help="layer copies cycled per graph pass")
    ap.add_argument("--workload", default="qwen3-30b-a3b")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--main-budget-only", action="store_true",
                    help="time only the 17.8%% budget (profiling runs)")
    ap.add_argument("--no-high-budget", action="store_true",
                    help="skip the 28.7%% budget (expected-error ranking, whole sketch)")
    ap.add_argument("--no-c5", action="store_true",
                    help="skip the Qwen3-235B-A22B-shaped layer at batch 8")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy, the reference kernel for "
                         "scaling FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--leg", choices=["k756", "k445", "dense", "b4", "shared4", "high", "c5", "q4"],
                    help="time one leg only and print its figures (profiling runs: one configuration "
                         "per counter pass)")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="summarise rocprofv3 CSV output under DIR as text and exit")
    ap.add_argument("--stack", action="store_true",
                    help="time only the 48-layer batch-1 decode step (route, decode, residual "
                         "per layer, captured as one HIP graph); prints its own JSON line")
    ap.add_argument("--no-q4", action="store_true",
                    help="skip the reader over the layer's 4-bit checkpoint")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 48-layer batch-1 decode step in the main line")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def copy_calibration(torch):
    """A plain elementwise copy of known size: reads and writes COPY_BYTES each."""
    src = torch.randn(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def profile_summary(d):
    """Text summary of rocprofv3 CSV output (kernel stats and FETCH_SIZE /
    WRITE_SIZE per dispatch) found under directory d."""
    import csv
    import glob

    def short(name):
        name = name.replace("(anonymous namespace)::", "").replace("cfr::", "")
        return name.split("(")[0]

    names = {"k_screen": "screen", "k_select": "select", "k_reduce": "reduce", "k_dense": "dense",
             "k_bscore": "bscore", "k_btopk": "btopk", "k_bact": "bact", "k_bdown": "bdown",
             "k_route": "route"}

    def ours(k):  # the decode-time kernels of the library
        return k.split("<")[0].split()[-1] in names

    lines = [f"device sources (csrc/*.hip, csrc/*.h) SHA-256: {source_digest()}"]
    traffic = {}
    for f in sorted(set(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))):
        lines.append(f"kernel stats: {os.path.relpath(f, d)}")
        lines.append(f"{'kernel':<44} {'calls':>7} {'avg us':>9} {'min us':>9} {'max us':>9} {'% time':>7}")
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if not ours(short(r["Name"])):
                    continue
                lines.append(f"{short(r['Name'])[:44]:<44} {int(r['Calls']):>7} "
                             f"{float(r['AverageNs']) / 1e3:>9.2f} {float(r['MinNs']) / 1e3:>9.2f} "
                             f"{float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>7.2f}")
    for f in sorted(set(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))):
        acc = {}
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (short(r["Kernel_Name"]), int(r["Grid_Size"]), r["Counter_Name"])
                a = acc.setdefault(key, [0.0, 0])
                a[0] += float(r["Counter_Value"])
                a[1] += 1
        lines.append(f"counters: {os.path.relpath(f, d)} (average per dispatch; FETCH_SIZE and "
                     "WRITE_SIZE in KiB; one line per kernel and grid size in threads)")
        for (k, g, c), (tot, n) in sorted(acc.items()):
            if ours(k):
                lines.append(f"  {k[:44]:<44} grid {g:>8} {c:<12} dispatches {n:>6}  avg {tot / n:>14.1f}")
        # the copy reference is the largest elementwise kernel of the run
        copy = [(k, c, tot / n) for (k, g, c), (tot, n) in acc.items()
                if "elementwise" in k.lower() and tot / n > 0.25 * (COPY_BYTES >> 10)]
        for k, c, v in copy:
            ratio = v * 1024 / COPY_BYTES
            scale = 1 / ratio if ratio else float("nan")
            lines.append(f"  copy reference {k[:40]} {c}: {v:.0f} KiB for {COPY_BYTES >> 10} KiB "
                         f"moved -> scale {scale:.4f}")
            traffic[c + "_scale"] = round(scale, 4)
        best = {}
        for (k, g, c), (tot, n) in acc.items():
            name = names.get(k.split("<")[0].split()[-1])
            if not name:
                continue
            ent = traffic.setdefault("kernels", {}).setdefault(name, {})
            # the grid launched most often stands for the kernel
            if best.get((name, c), (0, 0))[0] < n:
                best[(name, c)] = (n, g)
                ent["grid"] = g
                ent["fetch_kib" if c == "FETCH_SIZE" else "write_kib"] = round(tot / n, 1)
    print("\n".join(lines))
    traffic = {"source_sha256": source_digest(),
               "fetch_scale": traffic.get("FETCH_SIZE_scale"), "write_scale": traffic.get("WRITE_SIZE_scale"),
               "kernels": traffic.get("kernels", {})}
    with open(os.path.join(d, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1)


def graph_time(torch, readers, X, IDS, W, k, steps, warmup, fn="decode", Y=None, spread=None):
    """Capture one pass over all copies in a graph; return microseconds per step.
    With spread (a dict), also the median and 90th percentile of the per-pass
    averages (an event after every replay).  fn: "decode", "dense", or a
    layer step on copies built with router weights, on the residual stream
    x = Y[i]: "shared" (the batch-shared decode, k a list with one budget
    per copy), "route" (routing of RMSNorm(x) alone), "layer" (that routing,
    then the decode of the normed token, its output added to x in the
    decode's last kernel), "layer_dense" (the same with the dense block); IDS
    and W are then the routing's outputs."""
    L = len(readers)
    s = torch.cuda.Stream()
    if Y is None:
        Y = torch.empty((L, X.shape[1], X.shape[-1]), dtype=torch.float32, device=X.device)
    Hn = torch.empty_like(Y) if fn in ("route", "layer", "layer_dense") else None

    def one_pass():
        for i, r in enumerate(readers):
            if fn == "decode":
                r.decode(X[i], IDS[i], W[i], k, out=Y[i])
            elif fn == "shared":
                r.decode_shared(X[i], IDS[i], W[i], k[i], out=Y[i])  # k: one budget per copy
            elif fn == "dense":
                r.dense(X[i], IDS[i], W[i], out=Y[i])
            else:
                # x <- x + block(RMSNorm(x)) on the residual stream Y[i]
                r.route(Y[i], IDS[i], W[i], norm_out=Hn[i], norm_eps=1e-6)
                if fn == "layer":
                    r.decode(Hn[i], IDS[i], W[i], k, out=Y[i], residual=Y[i])
                elif fn == "layer_dense":
                    r.dense(Hn[i], IDS[i], W[i], out=Y[i], residual=Y[i])

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        one_pass()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        one_pass()
    torch.cuda.synchronize()
    # at least MIN_PASSES passes and MIN_DECODES decodes, whatever --steps says
    reps = max(MIN_PASSES, -(-steps // L), -(-MIN_DECODES // L))
    wreps = max(1, -(-warmup // L))
    with torch.cuda.stream(s):
        for _ in range(wreps):
            g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(s)
        for i in range(reps):
            g.replay()
            ev[i + 1].record(s)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[-1])
    if spread is not None:
        per = sorted(1000.0 * ev[i].elapsed_time(ev[i + 1]) / L for i in range(reps))
        spread["median"] = round(per[len(per) // 2], 3)
        spread["p90"] = round(per[min(len(per) - 1, int(0.9 * len(per)))], 3)
        spread["passes"] = reps
    del g
    return 1000.0 * total_ms / (reps * L), reps * L, wreps * L


def shared_leg(torch, cfg, readers, X, IDS, W, ids_host, k_token, shape, args):
    """The batch-shared decode on every copy's batch, each at k = k_token
    times (distinct experts of the batch) / top: microseconds per token, the
    library's count of the bytes one call reads (averaged over the first
    eight copies) and its rate."""
    from calibration_free_channel_amd import read_bytes_shared
    B = X.shape[1]
    ks = [int(round(k_token * np.unique(ids_host[i]).size / shape.top)) for i in range(len(readers))]
    us, _, _ = graph_time(torch, readers, X, IDS, W, ks, min(args.steps, 400), args.warmup, fn="shared")
    nb = []
    for i in range(min(8, len(readers))):
        dbg = readers[i].decode_debug(X[i], IDS[i], W[i], 0)  # the screened coordinates
        nb.append(read_bytes_shared(cfg, ids_host[i], dbg["sel"].cpu().numpy(), ks[i])["total"])
    bytes_call = float(np.mean(nb))
    return {"k_mean": round(float(np.mean(ks)), 1), "us_per_token": round(us / B, 3),
            "bytes_per_call": int(bytes_call), "GBps": round(bytes_call / us / 1e3, 1)}


def stage_times(torch, readers, X, IDS, W, k, steps, warmup):
    """Average duration of each decode kernel: the kernel launched alone, back
    to back over all layer copies in one HIP graph, timed with HIP events on
    the replay stream; returns {stage: microseconds per launch}.  Stage order
    keeps every launch meaningful: the screen is timed first (its sums pile
    up), a reduce pass clears them, a real screen pass fills them, then the
    select (which only reads them) and the reduce (which clears them)."""
    L = len(readers)
    s = torch.cuda.Stream()
    Y = torch.empty((L, X.shape[1], X.shape[-1]), dtype=torch.float32, device=X.device)

    def one_pass(stage):
        for i, r in enumerate(readers):
            r.decode_stage(stage, X[i], IDS[i], W[i], k, out=Y[i])

    def timed(stage):
        g = torch.cuda.CUDAGraph()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            one_pass(stage)
        torch.cuda.synchronize()
        reps = max(MIN_PASSES, -(-steps // L), -(-MIN_DECODES // L))
        with torch.cuda.stream(s):
            for _ in range(max(1, -(-warmup // L))):
                g.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        del g
        return 1000.0 * e0.elapsed_time(e1) / (reps * L)

    out = {"screen": timed(0)}
    with torch.cuda.stream(s):
        one_pass(2)
        one_pass(0)
    torch.cuda.synchronize()
    out["select"] = timed(1)
    out["reduce"] = timed(2)
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qwen3-30b-a3b_k756.json")
KERNEL_DIR = os.path.join(ROOT, "calibration_free_channel_amd", "csrc")


def source_digest():
    """SHA-256 over the device sources (every .hip and .h of the library, by
    name), so that counters taken on other kernels are not used."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(KERNEL_DIR, "*.hip")) + glob.glob(os.path.join(KERNEL_DIR, "*.h"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes(kernel):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE / WRITE_SIZE
    counter summary, each counter scaled by what it reads for a plain copy of
    known size; None when there is none, or when the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest() or kernel not in t.get("kernels", {}):
        return None
    c = t["kernels"][kernel]
    return int(round(1024.0 * (c["fetch_kib"] * t["fetch_scale"] + c["write_kib"] * t["write_scale"])))


def _cpu_model():
    """The host CPU's model name, from /proc/cpuinfo, else lscpu."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return None


def _host_cpus():
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(wl, layer, X, IDS, W, ks, seconds):
    """The oracle's float64 decode on the host, per token, at each budget in
    ks (the sample split evenly between them): on every BLAS thread it uses,
    then on one thread (a shorter sample) at the first budget."""
    from oracle import OracleReader
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
        threads = _host_cpus()
    s = wl.shape
    t = time.time()
    o = OracleReader(s.hidden, s.n_experts, s.inter, s.top, layer["gate"], layer["up"],
                     layer["down"], rot_seed=wl.rot_seed)
    log(f"oracle built in {time.time() - t:.1f}s (not timed)")

    def run(k, budget):
        n = 0
        t0 = time.perf_counter()
        while True:
            i = n % X.shape[0]
            o.decode(X[i, 0], IDS[i, 0], W[i, 0], k)
            n += 1
            el = time.perf_counter() - t0
            if (el >= budget and n >= 8) or n >= 4096:
                return n, el

    by_k = {}
    for k in ks:
        n, el = run(k, seconds / len(ks))
        by_k[f"k={k}"] = {"value": round(1e6 * el / n, 1), "tokens": n, "seconds": round(el, 1)}
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n1, el1 = run(ks[0], seconds / 4)
        one = {"value": round(1e6 * el1 / n1, 1), "k": ks[0], "tokens": n1, "seconds": round(el1, 1)}
    main = by_k[f"k={ks[0]}"]
    return {"value": main["value"], "unit": "us/token", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{main['tokens']} batch-1 tokens of the {wl.name} layer at k={ks[0]}, float64 "
                      f"numpy decode only (load-time build excluded), {main['seconds']}s of CPU work; "
                      "the other budgets on samples of the same length",
            "by_k": by_k, "single_core": one, "cpu_model": _cpu_model(), "host_cpus": _host_cpus()}


def stack_48l(steps, warmup):
    """The 48-layer stack of Qwen3-30B-A3B-shaped layers (independent weights
    per layer) as one batch-1 decode step: per layer h = RMSNorm(x) (unit
    weights, fused into the library's routing), the library routes h and
    decodes it at k = 756, adding the output to the residual stream x in its
    last kernel (x += y); the whole step is captured as one HIP graph
    and replayed, each replay from the same x0.  The dense BF16 block in the
    same chain is timed the same way, and so are the 48 routings alone."""
    import torch

    from calibration_free_channel_amd import Config, Reader, read_bytes
    from synth import make_layer, make_tokens, workload

    wl = workload("qwen3-30b-a3b-48l")
    s = wl.shape
    k = wl.ks[0]
    cfg = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top, rank=s.rank,
                 n_screen=s.n_screen, max_batch=1, rot_seed=wl.rot_seed)
    readers = []
    t = time.time()
    for l in range(wl.n_layers):
        L = make_layer(wl, layer=l)  # independent weights per layer
        readers.append(Reader.build(cfg, L["gate"], L["up"], L["down"], L["router"]))
        del L
        if l % 8 == 7:
            log(f"{l + 1} layers built ({time.time() - t:.0f}s)")
    torch.cuda.synchronize()
    x0 = torch.from_numpy(make_tokens(wl, 1)).cuda()
    x, h = torch.empty_like(x0), torch.empty_like(x0)
    ids = torch.empty((1, s.top), dtype=torch.int32, device="cuda")
    w = torch.empty((1, s.top), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()

    def one_step(mode):
        x.copy_(x0)
        for r in readers:
            r.route(x, ids, w, norm_out=h, norm_eps=1e-6)
            if mode == "route":
                continue
            # x += block(h): the residual is added in the block's last kernel
            if mode == "dense":
                r.dense(h, ids, w, out=x, residual=x)
            else:
                r.decode(h, ids, w, k, out=x, residual=x)

    def timed(mode, steps, warmup, spread=None):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            one_step(mode)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            one_step(mode)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            for _ in range(warmup):
                g.replay()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            ev[0].record(st)
            for i in range(steps):
                g.replay()
                ev[i + 1].record(st)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[-1])
        if spread is not None:
            per = sorted(1000.0 * ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
            spread["median"] = round(per[len(per) // 2], 2)
            spread["p90"] = round(per[min(steps - 1, int(0.9 * steps))], 2)
        del g
        return 1000.0 * ms / steps

    steps = max(MIN_PASSES, min(steps, 200))
    warm = max(2, min(warmup, 20))
    spread = {}
    us = timed("reader", steps, warm, spread)
    xr = x.clone()
    dense_us = timed("dense", steps, warm)
    route_us = timed("route", steps, warm)
    rb = read_bytes(cfg, k)
    per_layer = rb["total"] + s.n_experts * s.hidden * 2  # reader reads + router weights
    out = {
        "metric": "48-layer batch-1 decode step us (route, reader at 17.8% reads, residual)",
        "value": round(us, 2), "unit": "us/step", "n_gpus": 1, "steps": steps, "warmup": warm,
        "higher_is_better": False, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "48-layer stack of qwen3-30b-a3b-shaped layers, batch 1, k=756, "
                               "pre-norm (RMSNorm, unit weights) and residual",
                   "layers": wl.n_layers, "timing": "one hip graph per step, replayed"},
        "us_per_layer": round(us / wl.n_layers, 3),
        "per_step_median_us": spread["median"], "per_step_p90_us": spread["p90"],
        "bytes_per_step": per_layer * wl.n_layers,
        "achieved_GBps": round(per_layer * wl.n_layers / us / 1e3, 1),
        "dense_bf16_us_per_step": round(dense_us, 2),
        "norm_and_route_us_per_step": round(route_us, 2),
        "speedup_vs_dense": round(dense_us / us, 3),
        "final_x_finite": bool(torch.isfinite(xr).all().item()),
    }
    for r in readers:
        r.close()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.profile_summary:
        profile_summary(args.profile_summary)
        return
    if args.stack:
        if args.gpus != 1:
            print("bench.py --stack runs on one GPU only.", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(stack_48l(args.steps, args.warmup)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs the single-GPU reader only; --gpus {args.gpus} is not supported "
              "(the multi-GPU expert-parallel split is a design note, not a built path).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from calibration_free_channel_amd import RANK_EXPECTED_ERROR, Config, Reader, read_bytes, read_bytes_batch
    from synth import make_layer, make_routing_inputs, make_tokens, workload

    wl = workload(args.workload)
    s = wl.shape
    k_main = wl.ks[0]
    k_low = wl.ks[1] if len(wl.ks) > 1 else None
    L = args.layers
    t = time.time()
    layer = make_layer(wl)
    log(f"weights generated in {time.time() - t:.1f}s")
    cfg = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                 rank=s.rank, n_screen=s.n_screen, max_batch=4, rot_seed=wl.rot_seed)
    t = time.time()
    # with the router's weights (for the layer-step leg; the decode never reads them)
    base = Reader.build(cfg, layer["gate"], layer["up"], layer["down"], layer["router"])
    log(f"reader built in {time.time() - t:.1f}s")
    readers = [base] + [base.clone() for _ in range(L - 1)]
    torch.cuda.synchronize()
    log(f"{L} layer copies resident")

    Xh = make_tokens(wl, L).reshape(L, 1, s.hidden)
    IDh, Wh = make_routing_inputs(wl, L)
    X = torch.from_numpy(Xh).cuda()
    IDS = torch.from_numpy(IDh.reshape(L, 1, s.top)).cuda()
    W = torch.from_numpy(Wh.reshape(L, 1, s.top)).cuda()

    def on(name):  # this leg runs: every leg by default, else the one asked for
        return args.leg is None or args.leg == name

    full = args.leg is None and not args.main_budget_only
    res = {}
    ks = ([k_main] if on("k756") else []) + \
        ([k_low] if k_low and ((args.leg is None and not args.main_budget_only) or args.leg == "k445") else [])
    for k in ks:
        spread = {}
        us, nsteps, nwarm = graph_time(torch, readers, X, IDS, W, k, args.steps, args.warmup, spread=spread)
        rb = read_bytes(cfg, k)
        stages = stage_times(torch, readers, X, IDS, W, k, min(args.steps, 400), args.warmup)
        res[k] = {"us": us, "steps": nsteps, "warmup": nwarm, "bytes": rb, "stages": stages, "spread": spread}
        log(f"k={k}: {us:.2f} us/token, {rb['total'] / us / 1e3:.1f} GB/s counted; stages "
            + ", ".join(f"{n}={v:.1f}" for n, v in stages.items()))
    dense_us = None
    if not args.no_dense and on("dense"):
        dense_us, _, _ = graph_time(torch, readers, X, IDS, W, 0, min(args.steps, 400),
                                    args.warmup, fn="dense")
        log(f"dense BF16 block: {dense_us:.2f} us/token")

    # one batch-1 layer step per copy: route RMSNorm(x) (the library's fused
    # pre-norm), decode the normed token with the residual added in the
    # decode's last kernel; the dense block the same way; the routing alone
    layer_step = {}
    if full:
        IDr = torch.empty_like(IDS)
        Wr = torch.empty_like(W)
        Xr = X.clone()  # the residual stream, carried on over the replays
        for name, fn in (("reader", "layer"), ("dense", "layer_dense"), ("route", "route")):
            us_l, _, _ = graph_time(torch, readers, X, IDr, Wr, k_main, min(args.steps, 400), args.warmup,
                                    fn=fn, Y=Xr)
            layer_step[f"{name}_us"] = round(us_l, 3)
        layer_step["speedup_vs_dense"] = round(layer_step["dense_us"] / layer_step["reader_us"], 3)
        layer_step["residual_finite"] = bool(torch.isfinite(Xr).all())
        log("layer step, us: " + ", ".join(f"{n}={v}" for n, v in layer_step.items()))

    # batch 4 (per-token routing and top-k), the configuration's batched case:
    # µs per token = µs per call / 4
    batch4 = {}
    if full or args.leg in ("b4", "shared4"):
        X4 = torch.from_numpy(make_tokens(wl, 4 * L, seed_offset=7).reshape(L, 4, s.hidden)).cuda()
        I4h, W4h = make_routing_inputs(wl, 4 * L, seed_offset=7)
        I4 = torch.from_numpy(I4h.reshape(L, 4, s.top)).cuda()
        W4 = torch.from_numpy(W4h.reshape(L, 4, s.top)).cuda()
        for k in ([k_main] + ([k_low] if k_low else [])) if args.leg != "shared4" else []:
            us4, _, _ = graph_time(torch, readers, X4, I4, W4, k, min(args.steps, 400), args.warmup)
            batch4[f"k={k}"] = round(us4 / 4, 3)
            dbg = {n: v.cpu().numpy() for n, v in readers[0].decode_debug(X4[0], I4[0], W4[0], k).items()}
            ub4 = read_bytes_batch(cfg, I4[0].cpu().numpy(), dbg["sel"], dbg["kept"], k)["total"]
            batch4[f"k={k}_union_GBps"] = round(ub4 / us4 / 1e3, 1)
            batch4[f"k={k}_stages_us_per_call"] = {
                n: round(v, 2) for n, v in stage_times(torch, readers, X4, I4, W4, k, min(args.steps, 400),
                                                       args.warmup).items()}
        if not args.no_dense and args.leg != "shared4":
            us4, _, _ = graph_time(torch, readers, X4, I4, W4, 0, min(args.steps, 400), args.warmup,
                                   fn="dense")
            batch4["dense"] = round(us4 / 4, 3)
        # batch-shared selection: one top-k per call over the call's distinct
        # experts, at the per-token budget's share of the union
        for k in ([k_main] + ([k_low] if k_low else [])) if args.leg != "b4" else []:
            sh = shared_leg(torch, cfg, readers, X4, I4, W4, I4h.reshape(L, 4, s.top), k, s, args)
            batch4[f"shared_k={k}"] = sh
        log("batch 4, us/token: " + ", ".join(f"{n}={v}" for n, v in batch4.items()))

    # 28.7% and up: the whole sketch with the expected-error ranking, on copies
    # of a reader built for it (the resident bytes are the same layout)
    high = None
    if (full and not args.no_high_budget) or args.leg == "high":
        for r in readers[1:]:
            r.close()
        readers = readers[:1]
        torch.cuda.empty_cache()
        cfg_h = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top,
                       rank=s.rank, n_screen=128, max_batch=4, rot_seed=wl.rot_seed,
                       ranking=RANK_EXPECTED_ERROR)
        k_h = min(range(s.top * s.inter + 1),
                  key=lambda kk: abs(read_bytes(cfg_h, kk)["total"] / read_bytes(cfg_h, kk)["dense"] - 0.287))
        base_h = Reader.build(cfg_h, layer["gate"], layer["up"], layer["down"])
        readers_h = [base_h] + [base_h.clone() for _ in range(L - 1)]
        torch.cuda.synchronize()
        us_h, _, _ = graph_time(torch, readers_h, X, IDS, W, k_h, min(args.steps, 400), args.warmup)
        st_h = stage_times(torch, readers_h, X, IDS, W, k_h, min(args.steps, 400), args.warmup)
        rb_h = read_bytes(cfg_h, k_h)
        high = {"k": k_h, "us": us_h, "bytes": rb_h, "stages": st_h}
        log(f"28.7% (k={k_h}, whole sketch, expected-error ranking): {us_h:.2f} us/token, "
            f"{rb_h['total'] / us_h / 1e3:.1f} GB/s counted; stages "
            + ", ".join(f"{n}={v:.1f}" for n, v in st_h.items()))
        for r in readers_h:
            r.close()

    # the Qwen3-235B-A22B-shaped layer at batch 8 (per-token routing and top-k)
    c5 = None
    if (full and not args.no_c5) or args.leg == "c5":
        for r in readers[1:]:
            r.close()
        readers = readers[:1]
        torch.cuda.empty_cache()
        w5 = workload("qwen3-235b-a22b")
        s5 = w5.shape
        t = time.time()
        l5 = make_layer(w5)
        cfg5 = Config(hidden=s5.hidden, n_experts=s5.n_experts, inter=s5.inter, top=s5.top, rank=s5.rank,
                      n_screen=s5.n_screen, max_batch=8, rot_seed=w5.rot_seed)
        b5 = Reader.build(cfg5, l5["gate"], l5["up"], l5["down"])
        del l5
        L5 = 8
        r5 = [b5] + [b5.clone() for _ in range(L5 - 1)]
        torch.cuda.synchronize()
        log(f"qwen3-235b-a22b layer built and copied in {time.time() - t:.1f}s")
        X5 = torch.from_numpy(make_tokens(w5, 8 * L5).reshape(L5, 8, s5.hidden)).cuda()
        i5, g5 = make_routing_inputs(w5, 8 * L5)
        I5 = torch.from_numpy(i5.reshape(L5, 8, s5.top).astype(np.int32)).cuda()
        W5 = torch.from_numpy(g5.reshape(L5, 8, s5.top).astype(np.float32)).cuda()
        k5 = w5.ks[0]
        us5, _, _ = graph_time(torch, r5, X5, I5, W5, k5, min(args.steps, 200), args.warmup)
        st5 = stage_times(torch, r5, X5, I5, W5, k5, min(args.steps, 200), args.warmup)
        ud5 = None
        if not args.no_dense:
            ud5, _, _ = graph_time(torch, r5, X5, I5, W5, 0, min(args.steps, 200), args.warmup, fn="dense")
        sh5 = shared_leg(torch, cfg5, r5, X5, I5, W5, i5.reshape(L5, 8, s5.top), k5, s5, args)
        rb5 = read_bytes(cfg5, k5)
        dbg = {n: v.cpu().numpy() for n, v in r5[0].decode_debug(X5[0], I5[0], W5[0], k5).items()}
        ub5 = read_bytes_batch(cfg5, I5[0].cpu().numpy(), dbg["sel"], dbg["kept"], k5)["total"]
        c5 = {"k": k5, "batch": 8, "us_per_token": round(us5 / 8, 3),
              "union_bytes_per_call": ub5, "union_GBps": round(ub5 / us5 / 1e3, 1),
              "stages_us_per_call": {n: round(v, 2) for n, v in st5.items()},
              "read_pct_of_dense": round(100.0 * rb5["total"] / rb5["dense"], 2),
              # per-token counted bytes summed over the batch (experts routed by
              # several tokens are counted once per token: an upper bound on the
              # distinct bytes)
              "sum_of_token_bytes_GBps": round(8 * rb5["total"] / us5 / 1e3, 1),
              "dense_us_per_token": None if ud5 is None else round(ud5 / 8, 3),
              "speedup_vs_dense": None if ud5 is None else round(ud5 / us5, 3),
              "shared": sh5}
        log(f"qwen3-235b-a22b batch 8, k={k5}: {us5 / 8:.2f} us/token"
            + ("" if ud5 is None else f", dense {ud5 / 8:.2f} us/token"))
        for r in r5:
            r.close()

    # a 4-bit checkpoint of the same layer (exact rows in 4 bits, sketch
    # unchanged): the reader at k = 756 and at the k whose counted reads are
    # 18.9% of the BF16 routed bytes, beside the 4-bit dense block
    q4 = None
    if (full and not args.no_q4) or args.leg == "q4":
        for r in readers[1:]:
            r.close()
        readers = readers[:1]
        torch.cuda.empty_cache()
        from synth import make_layer_q4
        t = time.time()
        lq = make_layer_q4(wl)
        cfg_q = Config(hidden=s.hidden, n_experts=s.n_experts, inter=s.inter, top=s.top, rank=s.rank,
                       n_screen=s.n_screen, max_batch=4, rot_seed=wl.rot_seed, exact_bits=4)
        bq = Reader.build_q4(cfg_q, lq["rows"])
        del lq
        rq = [bq] + [bq.clone() for _ in range(L - 1)]
        torch.cuda.synchronize()
        log(f"4-bit layer built and copied in {time.time() - t:.1f}s")
        bf16_dense = read_bytes(cfg, 0)["dense"]
        k189 = min(range(s.top * s.inter + 1),
                   key=lambda kk: abs(read_bytes(cfg_q, kk)["total"] / bf16_dense - 0.189))
        q4 = {}
        for kq in (k_main, k189):
            us_q, _, _ = graph_time(torch, rq, X, IDS, W, kq, min(args.steps, 400), args.warmup)
            rbq = read_bytes(cfg_q, kq)
            q4[f"k={kq}"] = {"us_per_token": round(us_q, 3), "read_bytes_per_token": rbq["total"],
                             "read_pct_of_bf16_dense": round(100.0 * rbq["total"] / bf16_dense, 2),
                             "achieved_GBps": round(rbq["total"] / us_q / 1e3, 1)}
        udq, _, _ = graph_time(torch, rq, X, IDS, W, 0, min(args.steps, 400), args.warmup, fn="dense")
        q4["dense_q4_us_per_token"] = round(udq, 3)
        q4["dense_q4_GBps"] = round(read_bytes(cfg_q, 0)["dense"] / udq / 1e3, 1)
        for kk in (k_main, k189):
            q4[f"k={kk}"]["speedup_vs_dense_q4"] = round(udq / q4[f"k={kk}"]["us_per_token"], 3)
        log("4-bit rows: " + json.dumps(q4))
        for r in rq:
            r.close()

    # the 48-layer stack (independent weights per layer) as one batch-1 step
    stack = None
    if full and not args.no_stack:
        for r in readers[1:]:
            r.close()
        readers = readers[:1]
        torch.cuda.empty_cache()
        t = time.time()
        stack = stack_48l(args.steps, args.warmup)
        log(f"48-layer step: {stack['value']} us/step (median {stack['per_step_median_us']}, "
            f"dense {stack['dense_bf16_us_per_step']}), {time.time() - t:.0f}s with the build")

    if args.copy_calibration:
        copy_calibration(torch)
        log(f"copy calibration: {COPY_BYTES >> 20} MiB read and written 4 times")
    if args.leg is not None:
        figures = {"k756": res, "k445": res, "dense": dense_us, "b4": batch4, "shared4": batch4,
                   "high": high, "c5": c5, "q4": q4}[args.leg]
        if args.leg in ("k756", "k445"):
            figures = {f"k={kk}": {"us_per_token": round(r["us"], 3), "stages_us": r["stages"]}
                       for kk, r in res.items()}
        print(json.dumps({"leg": args.leg, "figures": figures}), flush=True)
        for r in readers:
            r.close()
        return

    main_r = res[k_main]
    rb = main_r["bytes"]
    # algorithmic bytes of each kernel per launch (one token)
    stage_bytes = {
        "screen": rb["codes"] + rb["scales"] + rb["norms"],
        "select": rb["exact"] + rb["b"],
        "reduce": rb["u"],
    }
    dom = max(stage_bytes, key=lambda n: main_r["stages"].get(n, 0.0))
    dom_us = main_r["stages"][dom]
    achieved = stage_bytes[dom] / dom_us / 1e3  # GB/s
    traffic = traffic_bytes(dom)
    path_gbps = rb["total"] / main_r["us"] / 1e3

    cpu = None
    if not args.no_cpu_baseline and args.leg is None:
        cpu = cpu_baseline(wl, layer, Xh, IDh.reshape(L, 1, s.top), Wh.reshape(L, 1, s.top),
                           [k_main] + ([k_low] if k_low else []), args.cpu_seconds)
        log(f"cpu baseline: {cpu['by_k']} us/token on {cpu['cores']} threads ({cpu['cpu_model']})"
            + (f", {cpu['single_core']['value']} us/token on one" if cpu["single_core"] else ""))

    out = {
        "metric": METRIC,
        "value": round(main_r["us"], 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": main_r["steps"],
        "warmup": main_r["warmup"],
        "ms_per_step": round(main_r["us"] / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} routed-expert layer, batch 1, k={k_main} (17.8% reads)",
                   "hidden": s.hidden, "n_experts": s.n_experts, "inter": s.inter, "top": s.top,
                   "k": k_main, "rank": s.rank, "n_screen": s.n_screen, "batch": 1,
                   "weights": "bf16", "layer_copies_cycled": L, "timing": "hip graph replay"},
        "achieved_GBps": round(path_gbps, 1),
        "hbm_frac": round(path_gbps / HBM_PEAK_GBPS, 4),
        "read_bytes_per_token": rb["total"],
        "read_pct_of_dense": round(100.0 * rb["total"] / rb["dense"], 2),
        "budgets": {
            f"{100.0 * r['bytes']['total'] / r['bytes']['dense']:.1f}%": {
                "k": kk, "us_per_token": round(r["us"], 3),
                "per_pass_median_us": r["spread"].get("median"), "per_pass_p90_us": r["spread"].get("p90"),
                "achieved_GBps": round(r["bytes"]["total"] / r["us"] / 1e3, 1),
                "stages_us": {n: round(v, 2) for n, v in r["stages"].items()}}
            for kk, r in res.items()},
        "budget_28.7%": None if high is None else {
            "k": high["k"], "ranking": "expected_error", "n_screen": 128,
            "read_pct_of_dense": round(100.0 * high["bytes"]["total"] / high["bytes"]["dense"], 2),
            "us_per_token": round(high["us"], 3),
            "achieved_GBps": round(high["bytes"]["total"] / high["us"] / 1e3, 1),
            "speedup_vs_dense": None if dense_us is None else round(dense_us / high["us"], 3),
            "stages_us": {n: round(v, 2) for n, v in high["stages"].items()}},
        "dense_bf16_us_per_token": None if dense_us is None else round(dense_us, 3),
        "dense_achieved_GBps": None if dense_us is None else round(rb["dense"] / dense_us / 1e3, 1),
        "speedup_vs_dense": None if dense_us is None else round(dense_us / main_r["us"], 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": dom, "bytes_per_launch": stage_bytes[dom],
                     "us_per_launch": round(dom_us, 3),
                     "timing": "kernel alone, back to back over the layer copies in a HIP graph"},
        "batch4_us_per_token": batch4 or None,
        "layer_step_batch1": (dict(layer_step, what="per layer copy: route RMSNorm(x), decode it at k="
                                   f"{k_main}, output added to x in the decode's last kernel; dense: the same "
                                   "with the dense block; route: the routing alone")
                              if layer_step else None),
        "qwen3_235b_a22b_batch8": c5,
        "int4_exact_rows": q4,
        "stack_48l": None if stack is None else {
            kk: stack[kk] for kk in ("value", "unit", "steps", "us_per_layer", "per_step_median_us",
                                     "per_step_p90_us", "achieved_GBps", "dense_bf16_us_per_step",
                                     "norm_and_route_us_per_step", "speedup_vs_dense", "final_x_finite")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    for r in readers:
        r.close()


if __name__ == "__main__":
    main()
