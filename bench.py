#!/usr/bin/env python3
"""Benchmark of the sampling step on one MI355X: sampled rows/s and achieved HBM GB/s for
[B, V] logits -> token ids.

Default workload: B=256 x V=151936 bf16 logits ~ N(0, 0.5^2), per-row T ~ U[0.3, 1.5],
per-row seeds and offsets, HLG curve (m=1.25, w=1.5, beta_t=0.5, beta_h=1.0) fused with the
Gumbel-max draw in one launch. One step = one hs_sample call over the batch. Inputs are
resident in HBM before timing starts; five copies of the logits (389 MB, more than the
256 MB last-level cache) are used in turn so every step reads its logits from HBM.

Prints ONE JSON line on stdout (details on stderr). The CPU baseline is the double-precision
oracle timed on this host's cores on a bounded sample of the same rows.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("sampled rows/sec and achieved HBM GB/s (% of peak) for [B,V] logits → token "
          "ids")
HBM_PEAK_GBPS = 8000.0
# VALU lane-operations per second of MI355X at its nominal clock: 256 CUs x 4 SIMDs x 16 lanes
# x 2.4 GHz (no packed fp32). Reported beside the HBM roofline, not as it.
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# An algorithmic count of VALU operations per element and draw, for context only (the
# measured VALU-busy fraction comes from the SQ counters): Philox4x32-10 share 10 (10 rounds x
# 2 mul-hi/lo + 2 three-way xor, per 4 words), upcast 1, compare 1; plus, once per element
# with the curve on, the log-sum-exp's max / exponent-argument / exp / add (4).
OPS_PER_ELEMENT_DRAW = 12
OPS_PER_ELEMENT_LSE = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """A digest of the sampling kernels' code (comments and blank lines left out, so that a
    profile stays valid across edits of the comments only)."""
    import re
    h = hashlib.sha256()
    for f in ("hs_kernels.hip", "hs_kernels_scr.hip", "hs_kernels_pivot.hip",
              "hs_kernels_pivot_scr.hip", "hs_kernels_rows.hip", "hs_kernels_rows_scr.hip",
              "hs_sample_kernel.hpp", "hs_device.hpp", "hs_api.hip", "hs_internal.hpp"):
        with open(os.path.join(ROOT, "logit_transform_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(l.rstrip() for l in text.splitlines() if l.strip())
        h.update(text.encode())
    return h.hexdigest()[:16]


def load_profile(kind: str, name: str):
    """A committed rocprofv3 counter summary (profiles/<kind>_<name>.json), if it was taken on
    the current kernel sources; None otherwise."""
    p = os.path.join(ROOT, "profiles", "%s_%s.json" % (kind, name))
    if not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != kernel_source_digest():
        return None
    return d


def load_traffic(name: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary."""
    d = load_profile("traffic", name)
    return None if d is None else d.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s: float = 10.0, settings=None, filters=None, layout="plain"):
    """The oracle as it stands, all host cores, on the workload's rows: a first timed pass sizes
    the sample (the first rows, or whole passes over all rows repeated until about budget_s of
    work), then the sample is timed. Rows per second of the whole sample are reported."""
    from oracle import oracle as O
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    threads = int(os.environ["OMP_NUM_THREADS"])
    O.lib()
    n = min(w.B, max(threads, 8))

    def run(rows):
        if filters is not None:
            O.sample_filtered(w.logits[:rows], w.T[:rows], w.seed[:rows], w.offset[:rows],
                              K=w.K, top_k=filters[0], top_p=filters[1], layout=layout)
            return
        if settings is None:
            O.sample(w.logits[:rows], w.T[:rows], w.seed[:rows], w.offset[:rows], K=w.K,
                     mu=None if w.hlg is None else w.mu[:rows], hlg=w.hlg, layout=layout)
            return
        # the curve set per row: the oracle samples each row with its own setting
        import numpy as np
        for r in range(rows):
            h = settings[r]
            O.sample(w.logits[r:r + 1], w.T[r:r + 1], w.seed[r:r + 1], w.offset[r:r + 1],
                     K=w.K, mu=w.mu[r:r + 1] if h is not None and "pivot" not in h else None,
                     hlg=h, row_id=np.array([r], dtype=np.int64), layout=layout)

    run(n)   # first call: library and thread-pool start-up, untimed
    t0 = time.perf_counter()
    run(n)
    per_row = (time.perf_counter() - t0) / n
    rows = int(min(w.B, max(n, budget_s / max(per_row, 1e-9))))
    reps = 0
    t0 = time.perf_counter()
    while True:
        run(rows)
        reps += 1
        t1 = time.perf_counter()
        if t1 - t0 >= budget_s:
            break
    return {"value": reps * rows / (t1 - t0), "unit": "rows/s", "cores": threads,
            "kind": "oracle",
            "sample": "first %d of %d rows of the same workload (%d draw(s) each), %d pass(es), "
                      "%.1f s wall on %d OpenMP threads" % (rows, w.B, w.K, reps, t1 - t0,
                                                           threads)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_one_thread(cfg: int, rows: int, layout: str = "plain") -> None:
    """Child process (OMP_NUM_THREADS=1, no GPU): the oracle on the first rows of a workload;
    prints rows/s as JSON."""
    from oracle import oracle as O
    from synth import workloads as W
    w = W.WORKLOADS[cfg]()
    O.lib()
    def run():
        O.sample(w.logits[:rows], w.T[:rows], w.seed[:rows], w.offset[:rows], K=w.K,
                 mu=None if w.hlg is None else w.mu[:rows], hlg=w.hlg, layout=layout)
    run()
    t0 = time.perf_counter()
    run()
    dt = time.perf_counter() - t0
    print(json.dumps({"rows_per_s": rows / dt, "rows": rows, "seconds": dt}), flush=True)


def cpu_one_thread(cfg: int, rows: int, layout: str = "plain"):
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-one-thread",
                        str(cfg), str(rows), layout], env=env, capture_output=True, text=True,
                       timeout=300)
    if r.returncode != 0:
        return {"error": r.stderr.strip()[-200:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    if len(sys.argv) == 5 and sys.argv[1] == "--oracle-one-thread":
        oracle_one_thread(int(sys.argv[2]), int(sys.argv[3]), sys.argv[4])
        return
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4,
                    help="workload: 4 = the 256 x 151936 bf16 headline (default); 1, 2, 3, 5 "
                         "for the other workloads of the pages")
    ap.add_argument("--copies", type=int, default=5, help="rotating input copies (cold cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the streaming-read and Philox ceilings and the warm-cache run")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps one by one instead of replaying a HIP graph")
    ap.add_argument("--pivot", choices=("input", "top", "entropy", "median"), default="input",
                    help="the curve's pivot: given per row (default, the workload's mu), "
                         "top-anchored or entropy-anchored, computed in the kernel, or the "
                         "mass median, from the threshold kernel")
    ap.add_argument("--pivot-offset", type=float, default=6.0,
                    help="c of the top anchor (nats below the most probable token)")
    ap.add_argument("--per-row", action="store_true",
                    help="set the curve per row (hs_sample_rows), cycling over: off, given "
                         "pivot, top-anchored, entropy-anchored, with the workload's knobs")
    ap.add_argument("--top-k", type=int, default=0,
                    help="top-k filter on every row (turns the curve off; 0 = none)")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="top-p filter on every row (turns the curve off; 1 = none)")
    ap.add_argument("--layout", choices=("plain", "screened"), default="screened",
                    help="word layout of the random stream: screened (default: the leading 16 "
                         "bits of eight elements come from one Philox call) or plain (element i "
                         "takes word i & 3 of the call at counter word i >> 2); the other "
                         "layout is timed beside it (other_layout)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device copy of MIB MiB five "
                         "times (reference for scaling the memory-traffic counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the sampling step has no multi-GPU path in this "
              "build (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import logit_transform_amd as hs
    from synth import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes x 5" % n)
        return
    L = hs.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.config]()
    B, V, K = w.B, w.V, w.K
    settings = None
    filtered = args.top_k > 0 or args.top_p < 1.0
    if filtered:
        # the filters act on the curve-off path
        w.hlg = None
        w.mu = None
        w.name += ", curve off, top-k %d, top-p %g" % (args.top_k, args.top_p)
    if w.hlg is not None and args.pivot != "input":
        w.hlg = dict(w.hlg, pivot=args.pivot, pivot_offset=args.pivot_offset)
        w.name += ", pivot %s" % args.pivot + (" c=%g" % args.pivot_offset
                                               if args.pivot == "top" else "")
    if args.per_row:
        if w.hlg is None:
            print("--per-row needs a workload with the curve on", file=sys.stderr)
            sys.exit(2)
        base = {k: w.hlg[k] for k in ("m", "w", "beta_t", "beta_h")}
        cycle = [None, dict(base), dict(base, pivot="top", pivot_offset=args.pivot_offset),
                 dict(base, pivot="entropy")]
        settings = [cycle[r % len(cycle)] for r in range(B)]
        w.name += ", curve per row (off / given / top c=%g / entropy)" % args.pivot_offset
    log("workload:", w.name)

    copies = [w.logits.to(dev)]
    for _ in range(max(0, args.copies - 1)):
        copies.append(copies[0].clone())
    T = torch.from_numpy(w.T).to(dev)
    seed = torch.from_numpy(w.seed.view(np.int64)).to(dev)
    off = torch.from_numpy(w.offset.view(np.int64)).to(dev)
    given_pivot = w.hlg is not None and (settings is not None or
                                         w.hlg.get("pivot", "input") == "input")
    mu = torch.from_numpy(w.mu).to(dev) if given_pivot else None
    hp = None if settings is not None else hs._hlg_struct(w.hlg)
    rows = hs.hlg_rows(settings, dev) if settings is not None else None
    out = torch.empty((B, K), dtype=torch.int32, device=dev)
    ws = hs.workspace(B, V, K, w.dtype, w.hlg is not None, dev)
    structs = [hs._logits_struct(x) for x in copies]
    stream = hs._stream(dev)
    hp_ref = C.byref(hp) if hp is not None else None
    mu_ptr = mu.data_ptr() if mu is not None else None

    topk_t = torch.full((B,), args.top_k, dtype=torch.int32, device=dev)
    topp_t = torch.full((B,), args.top_p, dtype=torch.float32, device=dev)
    # the plain layout runs through hs_sample itself; the screened one needs hs_sample_ex
    opts = hs.SampleOpts(layout=hs.LAYOUTS[args.layout])
    opts_ref = C.byref(opts)

    def launch(i, s_):
        if filtered:
            rc = L.hs_sample_filtered(C.byref(structs[i % len(structs)]), T.data_ptr(),
                                      topk_t.data_ptr(), topp_t.data_ptr(), seed.data_ptr(),
                                      off.data_ptr(), K, out.data_ptr(), None, ws.data_ptr(),
                                      ws.numel(), opts_ref, s_)
            if rc != 0:
                raise hs.HsError(rc, "hs_sample_filtered")
            return
        if rows is not None:
            rc = L.hs_sample_rows(C.byref(structs[i % len(structs)]), T.data_ptr(), mu_ptr,
                                  rows.data_ptr(), seed.data_ptr(), off.data_ptr(), K,
                                  out.data_ptr(), None, ws.data_ptr(), ws.numel(), opts_ref, s_)
        elif args.layout == "plain":
            rc = L.hs_sample(C.byref(structs[i % len(structs)]), T.data_ptr(), mu_ptr, hp_ref,
                             seed.data_ptr(), off.data_ptr(), K, out.data_ptr(), ws.data_ptr(),
                             ws.numel(), s_)
        else:
            rc = L.hs_sample_ex(C.byref(structs[i % len(structs)]), T.data_ptr(), mu_ptr,
                                hp_ref, seed.data_ptr(), off.data_ptr(), K, out.data_ptr(),
                                None, ws.data_ptr(), ws.numel(), opts_ref, s_)
        if rc != 0:
            raise hs.HsError(rc, "hs_sample_rows" if rows is not None else "hs_sample")

    def step(i):
        launch(i, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ref_ids = out.clone()
    # Timed region: K steps back to back on the stream, bracketed by two events. The K launches
    # are captured once in a HIP graph (one kernel node per step, the input copies in turn) and
    # the graph is replayed, so the host's launch rate does not pace the GPU; --eager launches
    # them one by one instead.
    graph = None
    if not args.eager:
        try:
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream(dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                with torch.cuda.graph(graph, stream=side):
                    cap_stream = hs._stream(dev)
                    for i in range(args.steps):
                        launch(i, cap_stream)
            torch.cuda.current_stream(dev).wait_stream(side)
            # untimed replays until about 0.2 s of work has run: the GPU's clock ramps up
            # over the first milliseconds of sustained load, and the timed region measures
            # the steady state
            t_w = time.perf_counter()
            for _ in range(50):
                graph.replay()
                torch.cuda.synchronize()
                if time.perf_counter() - t_w > 0.2:
                    break
        except Exception as e:   # noqa: BLE001 -- report and time eagerly instead
            log("graph capture failed (%s); timing eager launches" % e)
            graph = None
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    t_all1.record()
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    total_ms = t_all0.elapsed_time(t_all1)
    ms_per_step = total_ms / args.steps
    if not torch.equal(out, ref_ids):
        raise RuntimeError("sampled ids changed between identical steps")
    # Kernel duration for the roofline: the same launches, each between its own pair of events
    # on the stream the kernel runs on (the events' own work stays outside the pairs).
    nk = min(args.steps, 200)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nk)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nk)]
    torch.cuda.synchronize()
    for i in range(nk):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    per_launch = sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))
    # The roofline takes the kernel's duration from the events around the timed region (one
    # launch per step, back to back); the per-launch pairs, which also time the events' own
    # work, are reported beside it.
    kern_ms = ms_per_step

    # Ceilings on the same shape, each timed as a graph of back-to-back launches: a plain
    # streaming read of the logits with the sampler's access pattern (the same rotating
    # copies), and the Philox4x32-10 word rate with no memory traffic; and the sampler itself
    # with one input copy (warm: resident in the last-level cache).
    ceilings = warm = other_layout = None
    if not args.no_ceilings and graph is not None:
        def graph_ms(fn, n):
            g = torch.cuda.CUDAGraph()
            side_ = torch.cuda.Stream(dev)
            side_.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side_):
                with torch.cuda.graph(g, stream=side_):
                    cs = hs._stream(dev)
                    for i in range(n):
                        fn(i, cs)
            torch.cuda.current_stream(dev).wait_stream(side_)
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        n_c = min(args.steps, 200)
        # the other word layout on the same inputs, timed the same way (rotating copies)
        other = "plain" if args.layout == "screened" else "screened"
        mine = args.layout
        args.layout = other
        opts.layout = hs.LAYOUTS[other]
        other_ms = graph_ms(launch, n_c)
        args.layout = mine
        opts.layout = hs.LAYOUTS[mine]
        other_layout = {"layout": other, "ms_per_step": other_ms,
                        "rows_per_s": B / (other_ms / 1e3)}
        warm_ms = graph_ms(lambda i, s_: launch(0, s_), n_c)
        warm = {"ms_per_step": warm_ms, "rows_per_s": B / (warm_ms / 1e3),
                "note": "one input copy, resident in the last-level cache"}
        M = C.CDLL(os.path.join(ROOT, "logit_transform_amd", "libhs_micro.so"))
        M.hs_micro_stream_max.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                          C.c_int64, C.c_void_p, C.c_void_p]
        M.hs_micro_stream_max_nt.argtypes = M.hs_micro_stream_max.argtypes
        M.hs_micro_philox_max.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int32,
                                          C.c_int32, C.c_void_p, C.c_void_p]
        groups = max(1, min(K, -(-2048 // B)))   # spread the draws over about 2048 blocks
        esz = w.logits.element_size()
        rowmax = torch.empty(B, dtype=torch.float32, device=dev)
        words = torch.empty(B * groups * 1024, dtype=torch.int32, device=dev)
        ceilings = {}

        def read_one(i, s_, fn=M.hs_micro_stream_max):
            x = copies[i % len(copies)]
            rc = fn(x.data_ptr(), hs._DTYPES[x.dtype], B, V, x.stride(0), rowmax.data_ptr(), s_)
            if rc != 0:
                raise RuntimeError("hs_micro_stream_max: %d" % rc)

        def read_one_nt(i, s_):
            read_one(i, s_, M.hs_micro_stream_max_nt)

        def philox_one(i, s_):
            rc = M.hs_micro_philox_max(seed.data_ptr(), B, V, K, groups, words.data_ptr(), s_)
            if rc != 0:
                raise RuntimeError("hs_micro_philox_max: %d" % rc)

        if (V * esz) % 16 == 0:
            st_ms = graph_ms(read_one, n_c)
            st_gbps = B * V * esz / (st_ms / 1e3) / 1e9
            ceilings["stream_read"] = {"ms": st_ms, "GB/s": st_gbps,
                                       "frac_of_peak": st_gbps / HBM_PEAK_GBPS,
                                       "pattern": "one 1024-thread block per row, 16-byte loads, "
                                                  "8 in flight per lane"}
            nt_ms = graph_ms(read_one_nt, n_c)
            nt_gbps = B * V * esz / (nt_ms / 1e3) / 1e9
            ceilings["stream_read_nt"] = {"ms": nt_ms, "GB/s": nt_gbps,
                                          "frac_of_peak": nt_gbps / HBM_PEAK_GBPS,
                                          "pattern": "the same with non-temporal loads, 4 in "
                                                     "flight per lane (best read measured)"}
            best_gbps = max(st_gbps, nt_gbps)
            ceilings["kernel_frac_of_stream_read"] = B * V * esz / (kern_ms / 1e3) / 1e9 / best_gbps
        if V % 4 == 0:
            ph_ms = graph_ms(philox_one, min(n_c, 50))
            ceilings["philox"] = {"ms": ph_ms, "words_per_s": B * V * K / (ph_ms / 1e3),
                                  "draws": K}
            ceilings["kernel_words_per_s"] = B * V * K / (kern_ms / 1e3)
            ceilings["kernel_frac_of_philox"] = ph_ms / kern_ms
        log("warm (one copy, cache-resident) %.4f ms/step; ceilings %s" % (warm_ms, ceilings))

    rows_per_s = B / (ms_per_step / 1e3)
    logit_bytes = B * V * w.logits.element_size()
    param_bytes = B * (4 + 8 + 8 + (4 if mu is not None else 0) + (32 if rows is not None else 0))
    alg_bytes = logit_bytes + param_bytes + 4 * B * K
    gbps = alg_bytes / (kern_ms / 1e3) / 1e9
    # the log-sum-exp runs for every row unless the whole batch is top-anchored
    lse_on = w.hlg is not None and (rows is not None or w.hlg.get("pivot", "input") != "top")
    ops = B * V * (OPS_PER_ELEMENT_DRAW * K + (OPS_PER_ELEMENT_LSE if lse_on else 0))
    tops = ops / (kern_ms / 1e3) / 1e12
    name = "k_sample_c%d" % args.config
    if args.layout != "plain":
        name += "_" + args.layout
    if args.pivot != "input" and w.hlg is not None:
        name += "_" + args.pivot
    if rows is not None:
        name += "_rows"
    if filtered:
        name += "_filtered"
    traffic = load_traffic(name)
    log("step %.4f ms (events over the timed region), wall %.4f ms/step; per-launch event "
        "pairs p10 %.4f p50 %.4f p90 %.4f ms"
        % (ms_per_step, (wall1 - wall0) * 1e3 / args.steps, per_launch[len(per_launch) // 10],
           per_launch[len(per_launch) // 2], per_launch[(9 * len(per_launch)) // 10]))
    log("HBM %.1f GB/s = %.1f%% of 8 TB/s (algorithmic bytes over the kernel time)"
        % (gbps, 100 * gbps / HBM_PEAK_GBPS))
    sq = load_profile("valu", name)

    rec = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name + ", %s word layout" % args.layout, "B": B, "V": V,
                   "K": K, "layout": args.layout,
                   "input_dtype": str(w.dtype).replace("torch.", ""),
                   "hlg": w.hlg is not None, "input_copies": len(copies),
                   "pivot": (None if w.hlg is None else
                             "per_row" if rows is not None else w.hlg.get("pivot", "input")),
                   "top_k": args.top_k if filtered else None,
                   "top_p": args.top_p if filtered else None,
                   "launch": "hip_graph" if graph is not None else "eager",
                   "algorithmic_bytes_per_step": alg_bytes},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": name, "kernel_ms": kern_ms,
                     "algorithmic_bytes": alg_bytes,
                     "launch_pair_ms_p50": per_launch[len(per_launch) // 2]},
        # The kernel is limited by its VALU issue rate, not by HBM. The busy fraction comes from
        # the committed SQ counters (SQ_ACTIVE_INST_VALU / (SQ_WAVE_CYCLES / 4) summed over the
        # dispatch, null when they were taken on other kernel sources); the operation count is
        # the algorithmic one above, at the nominal 2.4 GHz, for context.
        "valu": {"busy_frac": None if sq is None else sq.get("valu_busy_frac"),
                 "insts_per_wave": None if sq is None else sq.get("valu_insts_per_wave"),
                 "algorithmic_ops_per_step": ops, "algorithmic_T_ops_per_s": tops,
                 "nominal_peak_T_ops_per_s": ALU_PEAK_TOPS},
        "launch_ms": {"p10": per_launch[len(per_launch) // 10],
                      "p50": per_launch[len(per_launch) // 2],
                      "p90": per_launch[(9 * len(per_launch)) // 10],
                      "note": "each launch between its own pair of events"},
    }
    if K > 1:
        rec["draws_per_s"] = B * K / (ms_per_step / 1e3)
    if warm is not None:
        rec["warm"] = warm
        rec["other_layout"] = other_layout
    if ceilings:
        rec["ceilings"] = ceilings
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(
            w, settings=settings, filters=(args.top_k, args.top_p) if filtered else None,
            layout=args.layout)
        rec["cpu_baseline"]["cpu_model"] = cpu_model()
        if settings is None and args.pivot == "input" and not filtered:
            rec["cpu_baseline"]["one_thread"] = cpu_one_thread(
                args.config, 1 if args.config == 5 else 16, args.layout)
        log("cpu baseline:", rec["cpu_baseline"])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
