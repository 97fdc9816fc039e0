#!/usr/bin/env python3
"""Benchmark of the Hogwild! concurrent-attention decode step on one MI355X.

A step is one decode step of every worker over every layer the workload times
(for w8_32k each layer first appends one new token per worker: under a step
plan by default, hw_append_step + hw_concurrent_decode). A step of at least 8
layers is captured once as a HIP graph and replayed, as a serving loop runs its
decode step (--eager: every kernel launched from the host). Inputs are seeded synthetic
tensors already resident in HBM when a timed region starts. With --query-tokens K > 1 every worker queries K
tokens per step together (hw_concurrent_decode_tokens, causal).

Prints ONE JSON line. The headline workload (default w4_16k) gives `value`
(worker-steps/s) and `ms_per_step`: the median over --repeats timed regions of
--steps steps each, with the spread beside it. A second workload (default
w8_32k, the 8-worker case with appends) is timed the same way and reported
under its own key. Each carries a roofline object for the dominant kernel
(concurrent_decode: algorithmic bytes per launch / its average duration, from
start/stop HIP events that the kernel's own dispatch records on its stream
during a timed pass), the measured streaming-read ceiling of the same GPU and
the fp64 oracle's CPU rate on one full step of the same workload (one process
per host core, in a child process that never touches the GPU).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "concurrent-attn decode worker-steps/s and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
# The sources that decide what the decode launches run: the kernels, the launch-argument
# layout, and the host code that picks partitions, row blocks and kernel shapes.
KERNEL_SRCS = [os.path.join(ROOT, "shared_kv_cache_amd", "csrc", f)
               for f in ("hw_kernels.hip", "hw_internal.h", "hw_host.cpp")]
WORKLOADS = ["tiny_fp32", "w2_4k", "w4_16k", "w8_32k", "w4_128k_sinks"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed (string literals kept), so
    that a change to comments alone leaves the hash unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_concurrent_decode_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per launch \(fetch \+ write, scaled\):\s*`?([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def run_gpu(name, args, graph, plan):
    """Time one workload on cuda:0. Returns the measured figures (no JSON formatting)."""
    import numpy as np
    import torch

    from shared_kv_cache_amd import hogwild as H
    from shared_kv_cache_amd import workloads as W

    dev = torch.device("cuda", 0)
    kq = args.query_tokens
    grows = name == "w8_32k"
    plan = plan and grows and kq == 1
    fused = plan and not getattr(args, "unfused", False)
    steps, reps = args.steps, args.repeats
    # planned window: warm-up, the timed repeats, the kernel-event pass and its warm-up step,
    # graph warm-up
    total_steps = args.warmup + reps * steps + steps + 5
    extra = {"n_layers": args.layers} if args.layers > 0 else {}
    wl = W.make(name, steps=total_steps if grows else 0, **extra)
    n, hq, hkv, d, L = wl.n_workers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_layers
    kv_dt = torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32
    elem = 2 if wl.kv_dtype == "bf16" else 4

    t0 = time.time()
    cache = H.HogwildCache(
        n_layers=L, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, page_size=wl.page_size,
        n_pages=wl.n_pages, max_blocks=len(wl.blocks()) + 1, max_workers=n,
        max_position=wl.max_position, kv_dtype=wl.kv_dtype, page_seed=wl.page_seed,
        rope_theta=wl.theta, max_splits=512 if args.splits > 256 else 0,
        max_query_tokens=kq, device="cuda:0")
    blocks = wl.blocks()

    def gen(layer):
        ks, vs = zip(*(wl.kv(layer, b) for b in blocks))
        return layer, np.concatenate(ks), np.concatenate(vs)

    with ThreadPoolExecutor(max_workers=8) as ex:
        for layer, k, v in ex.map(gen, range(L)):
            kt = torch.from_numpy(k).to(dev).to(kv_dt)
            vt = torch.from_numpy(v).to(dev).to(kv_dt)
            cache.append(layer, blocks, [wl.lengths[b] for b in blocks], kt, vt)
    cache.set_views(wl.views(args.layout))
    if args.splits:
        H.hw_set_split(cache.ctx, args.splits)
    if plan:
        cache.plan_steps(total_steps, wl.inprogress, [1] * n)
    # Inputs in fixed device buffers, per layer: the queries and (growing workloads) the
    # step's new token of every worker, as a model's projections would leave them.
    q_dev = [torch.from_numpy(wl.q(layer) if kq == 1 else wl.q_tokens(layer, kq)).to(dev)
             for layer in range(L)]
    step_kv = None
    if grows:
        step_kv = [tuple(torch.from_numpy(x).to(dev).to(kv_dt) for x in wl.step_kv(layer, 1))
                   for layer in range(L)]
    outs = [torch.empty((n, kq, hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    lses = [torch.empty((n, kq, hq), dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s: {wl.name}, {L} layers, T={wl.total_tokens()}"
        f"{', step plan' if plan else ''}")

    cur = {"stream": torch.cuda.current_stream(dev).cuda_stream}

    def step():
        stream = cur["stream"]
        for layer in range(L):
            if grows:
                k, v = step_kv[layer]
                if plan and fused:   # the append runs inside the decode launch
                    H.hw_decode_step(cache.ctx, layer, k.data_ptr(), v.data_ptr(),
                                     q_dev[layer].data_ptr(), outs[layer].data_ptr(),
                                     lses[layer].data_ptr(), stream)
                    continue
                if plan:
                    H.hw_append_step(cache.ctx, layer, k.data_ptr(), v.data_ptr(), stream)
                else:
                    H.hw_append_kv(cache.ctx, layer, wl.inprogress, [1] * n, k.data_ptr(),
                                   v.data_ptr(), stream)
            if kq == 1:
                H.hw_concurrent_decode(cache.ctx, layer, q_dev[layer].data_ptr(),
                                       outs[layer].data_ptr(), lses[layer].data_ptr(), stream)
            else:
                H.hw_concurrent_decode_tokens(cache.ctx, layer, kq, q_dev[layer].data_ptr(),
                                              outs[layer].data_ptr(), lses[layer].data_ptr(), stream)

    done = {"steps": 0}

    def run_steps(k):
        for _ in range(k):
            if g is not None:
                g.replay()
            else:
                step()
        done["steps"] += k

    g = None
    run_steps(args.warmup)
    torch.cuda.synchronize()
    if graph:
        if grows and not plan:
            raise SystemExit("--graph on a growing workload needs the step plan (drop --no-plan)")
        # Capture one step; growing workloads take their positions from the plan's counters.
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            cur["stream"] = side.cuda_stream
            step()
        cur["stream"] = torch.cuda.current_stream(dev).cuda_stream
        torch.cuda.synchronize()
        run_steps(2)
        torch.cuda.synchronize()

    def tokens_now():
        # under a plan the host's lengths stay at the plan's start; the device has appended
        # one token per worker and layer per step since
        base = sum(H.hw_block_info(cache.ctx, b, 0)[0] for b in blocks)
        return base + (n * done["steps"] if plan else 0)

    # Timed regions: `reps` regions of `steps` steps each, uninstrumented.
    t_tok0 = tokens_now()
    ms = []
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(reps):
        torch.cuda.synchronize()
        ev0.record()
        run_steps(steps)
        ev1.record()
        torch.cuda.synchronize()
        ms.append(ev0.elapsed_time(ev1))
    t_tok1 = tokens_now()
    # Kernel pass: the same steps run eagerly, the decode kernels recording start/stop events
    # (after one eager step unrecorded: the first eager launches after the replays run slow).
    gsave, g = g, None
    run_steps(1)
    torch.cuda.synchronize()
    H.hw_debug_kernel_events(cache.ctx, steps * L)
    torch.cuda.synchronize()
    run_steps(steps)
    torch.cuda.synchronize()
    dec_ms = H.hw_debug_kernel_elapsed(cache.ctx)
    H.hw_debug_kernel_events(cache.ctx, 0)
    t_tok2 = tokens_now()
    g = gsave
    n_splits = H.hw_debug_resolve(cache.ctx, 0, n)["n_splits"] if kq == 1 else None
    if plan:
        cache.plan_end()
    cache.close()
    del cache, g
    torch.cuda.synchronize()

    med = pct(ms, 0.5) / steps
    avg_tokens = 0.5 * (t_tok0 + t_tok1) if grows else float(wl.total_tokens())
    kern_tokens = 0.5 * (t_tok1 + t_tok2) if grows else float(wl.total_tokens())
    io_bytes = n * kq * (hq * d * 4 * 2 + hq * 4)
    launch_bytes = avg_tokens * hkv * d * 2 * elem + io_bytes
    kern_launch_bytes = kern_tokens * hkv * d * 2 * elem + io_bytes
    append_bytes = (n * hkv * d * elem * 2 * 2) if grows else 0   # read + write new K and V
    step_bytes = L * (launch_bytes + append_bytes)
    dec_avg = float(np.mean(dec_ms))
    return {
        "wl": wl, "plan": plan, "fused": fused, "graph": graph, "ms_step": med,
        "spread": {"repeats": reps, "steps_per_repeat": steps,
                   "ms_per_step_min": round(min(ms) / steps, 5),
                   "ms_per_step_p10": round(pct(ms, 0.1) / steps, 5),
                   "ms_per_step_p90": round(pct(ms, 0.9) / steps, 5),
                   "ms_per_step_max": round(max(ms) / steps, 5)},
        "worker_steps": n / (med * 1e-3), "avg_tokens": avg_tokens,
        "step_bytes": step_bytes, "launch_bytes": kern_launch_bytes, "dec_avg_ms": dec_avg,
        "achieved": kern_launch_bytes / (dec_avg * 1e-3) / 1e9, "n_splits": n_splits,
        "elem": elem,
    }


def describe(r, args, layout):
    """Config and roofline objects of one run_gpu result."""
    wl = r["wl"]
    step_gbps = r["step_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    default_cfg = layout == "combined" and not args.splits and not args.layers
    profile_name = wl.name if args.query_tokens == 1 else f"{wl.name}_qt{args.query_tokens}"
    traffic = read_traffic(profile_name) if default_cfg else None
    config = {
        "workload": wl.name, "layout": layout, "workers": wl.n_workers, "q_heads": wl.n_q_heads,
        "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "layers": wl.n_layers,
        "tokens_per_layer": round(r["avg_tokens"], 1), "kv_dtype": wl.kv_dtype,
        "page_size": wl.page_size, "splits_per_head": r["n_splits"],
        "step_ideal_bytes": int(r["step_bytes"]), "step_GBps": round(step_gbps, 1),
        "step_frac_of_hbm_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "decode_kernel_us": round(r["dec_avg_ms"] * 1e3, 3),
        "per_layer_other_us": round(r["ms_step"] * 1e3 / wl.n_layers - r["dec_avg_ms"] * 1e3, 3),
        "appends_per_step": wl.n_layers if wl.name == "w8_32k" else 0,
        "query_tokens": args.query_tokens, "hip_graph": r["graph"], "step_plan": r["plan"],
        "append_fused_into_decode": r["fused"],
    }
    roofline = {"bound": "hbm", "achieved": round(r["achieved"], 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(r["achieved"] / HBM_PEAK_GBPS, 4),
                "traffic": traffic}
    return config, roofline


def stream_ceiling(sizes, reps=10):
    """Streaming-read ceiling: the library's plain read probe (16-byte streaming loads,
    every byte read once) over fresh windows of a 1 GiB buffer, so that no launch re-reads
    what the 256 MB last-level cache may still hold; median of `reps` launches timed by
    events of the kernel's own dispatch, best of two grid sizes."""
    import torch

    from shared_kv_cache_amd import hogwild as H

    dev = torch.device("cuda", 0)
    total = 1 << 30
    buf = torch.ones(total // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(1 << 14, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    points = []
    for nbytes in sizes:
        nb = nbytes // 256 * 256
        windows = max(1, total // nb)
        best = None
        for n_blocks in (4 * cus, 8 * cus):
            for r in range(2):      # warm-up launches
                H.hw_debug_stream_read(buf.data_ptr() + (r % windows) * nb, nb, sink.data_ptr(),
                                       n_blocks, stream)
            ms = sorted(H.hw_debug_stream_read(buf.data_ptr() + ((r + 2) % windows) * nb, nb,
                                               sink.data_ptr(), n_blocks, stream, timed=True)
                        for r in range(reps))
            gbps = nb / (ms[len(ms) // 2] * 1e-3) / 1e9
            if best is None or gbps > best["GBps"]:
                best = {"bytes": nb, "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                        "us": round(ms[len(ms) // 2] * 1e3, 2), "workgroups": n_blocks}
        points.append(best)
        log(f"stream read {nb} B: {best['GBps']} GB/s ({best['us']} us, {best['workgroups']} workgroups)")
    del buf, sink
    return {"kernel": "stream_read_kernel via hw_debug_stream_read", "points": points}


# ------------------------------------------------------------------ CPU baseline

def _oracle_layer(job):
    """One layer of the oracle on one thread (a pool worker): (layer, seconds of oracle time).
    The inputs are drawn before the clock starts."""
    name, layer, layout, kq, n_layers = job
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import hogwild_oracle as O
    from shared_kv_cache_amd import workloads as W

    wl = W.make(name, n_layers=n_layers)
    with threadpool_limits(limits=1):
        blocks = {b: tuple(x.astype(np.float64) for x in wl.kv(layer, b)) for b in wl.blocks()}
        q = (wl.q(layer) if kq == 1 else wl.q_tokens(layer, kq)).astype(np.float64)
        t0 = time.perf_counter()
        O.concurrent_attention(q, blocks, wl.views(layout), theta=wl.theta)
        return layer, time.perf_counter() - t0


def cpu_description():
    """The first processor's identification in /proc/cpuinfo: its model name as the kernel
    reports it (virtual machines may give only a family name), with vendor, family, model
    and stepping numbers."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if not ln.strip():
                    break                       # end of the first processor's entry
                k, _, v = ln.partition(":")
                fields.setdefault(k.strip(), v.strip())
    except OSError:
        return "unknown"
    ident = ", ".join(f"{k} {fields[k]}" for k in ("vendor_id", "cpu family", "model", "stepping")
                      if k in fields)
    return f"{fields.get('model name', 'unknown')} ({ident})" if ident else fields.get("model name", "unknown")


def cpu_baseline_child(name, layout, kq, procs):
    """Runs in a child process that never touches the GPU: the fp64 oracle, as it stands, on
    one full step of the workload (every layer, worker and query head), layer l on pool
    process l mod procs, each process single-threaded; the step's time is the busiest
    process's total. Then one layer alone on one thread."""
    import multiprocessing as mp

    from shared_kv_cache_amd import workloads as W

    wl = W.make(name)
    L = wl.n_layers
    model = cpu_description()
    one = _oracle_layer((name, 0, layout, kq, L))[1]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(processes=procs) as pool:
        res = pool.map(_oracle_layer, [(name, layer, layout, kq, L) for layer in range(L)],
                       chunksize=1)
    wall = time.perf_counter() - t0
    busy = [0.0] * procs
    for layer, sec in res:
        busy[layer % procs] += sec
    step_s = max(busy)
    rate = wl.n_workers / step_s
    return {"value": round(rate, 5), "unit": "worker-steps/s", "cores": procs, "kind": "oracle",
            "sample": f"one full step of {name}: all {L} layers, {wl.n_workers} workers "
                      f"({kq} query token(s) each), {wl.n_q_heads} query heads; fp64 numpy "
                      f"oracle, layer l on process l mod {procs}, one BLAS thread each; step time "
                      f"= the busiest process's oracle seconds ({step_s:.2f} s; pool wall "
                      f"{wall:.2f} s including input draws)",
            "cpu_model": model, "single_thread_s_per_layer": round(one, 3),
            "step_seconds": round(step_s, 3)}


def cpu_baseline(name, layout, kq):
    procs = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        procs = min(procs, int(os.environ["OMP_NUM_THREADS"]))
    procs = max(1, min(procs, 16))
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--workload", name,
           "--layout", layout, "--query-tokens", str(kq), "--cpu-procs", str(procs)]
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    t0 = time.time()
    out = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=900)
    if out.returncode != 0:
        log(out.stderr[-2000:])
        raise RuntimeError(f"cpu baseline child failed ({out.returncode})")
    res = json.loads(out.stdout.strip().splitlines()[-1])
    log(f"cpu oracle {name}: {res['value']} worker-steps/s on {res['cores']} processes "
        f"({time.time() - t0:.1f}s)")
    return res


# ------------------------------------------------------------------ main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="steps per timed region")
    ap.add_argument("--repeats", type=int, default=20, help="timed regions; the median is reported")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="w4_16k", choices=WORKLOADS)
    ap.add_argument("--extra-workload", default="w8_32k", choices=WORKLOADS + ["none"],
                    help="a second workload timed in the same run, reported under its own key")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB copy kernel (counter calibration)")
    ap.add_argument("--splits", type=int, default=0, help="force KV partitions per head")
    ap.add_argument("--layout", default="combined",
                    choices=["combined", "stepwise", "contiguous", "nosync"],
                    help="cache layout the views follow (combined: the method's own)")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer pools to rotate through (0: the workload's own count; 1 keeps one "
                         "layer's K/V resident in the last-level cache)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step's kernels from the host instead of replaying the "
                         "step captured once as a HIP graph (the default)")
    ap.add_argument("--graph", action="store_true", help=argparse.SUPPRESS)   # the default
    ap.add_argument("--no-plan", action="store_true",
                    help="growing workloads: host-planned appends (hw_append_kv) instead of a step plan")
    ap.add_argument("--unfused", action="store_true",
                    help="step plans: append (hw_append_step) and decode as two calls instead of "
                         "hw_decode_step, the append fused into the decode")
    ap.add_argument("--query-tokens", type=int, default=1,
                    help="query tokens per worker and step (several: one causal decode of all)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--cpu-procs", type=int, default=1, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.cpu_baseline_child:
        print(json.dumps(cpu_baseline_child(args.workload, args.layout, args.query_tokens,
                                            args.cpu_procs)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the concurrent-"
              "attention step here is single-GPU by design", file=sys.stderr)
        return 2
    if args.query_tokens < 1 or args.steps < 1 or args.repeats < 1:
        print("--query-tokens, --steps and --repeats must be at least 1", file=sys.stderr)
        return 2

    import torch

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x torch.mul(src, 1.0, out=dst), 1 GiB read + 1 GiB written each")

    plan = not args.no_plan
    def graphed(name):
        # A step of a few layers launches faster than a graph replays (tiny_fp32, one decode
        # launch: 9.3 us eager, 18 us replayed), so only steps of at least 8 layers are
        # replayed. A growing workload replays a captured step only under a step plan.
        from shared_kv_cache_amd import workloads as W
        grows = name == "w8_32k"
        many = (args.layers or W.make(name).n_layers) >= 8
        return not args.eager and many and (not grows or (plan and args.query_tokens == 1))

    head = run_gpu(args.workload, args, graphed(args.workload), plan)
    log(f"{args.workload}: median {head['ms_step']:.4f} ms/step over {args.repeats} x "
        f"{args.steps} steps; decode kernel {head['dec_avg_ms'] * 1e3:.2f} us")
    extra = None
    if args.extra_workload != "none" and args.extra_workload != args.workload:
        # the second workload the same way: growing ones under a step plan
        extra = run_gpu(args.extra_workload, args, graphed(args.extra_workload), plan)
        log(f"{args.extra_workload}: median {extra['ms_step']:.4f} ms/step; decode kernel "
            f"{extra['dec_avg_ms'] * 1e3:.2f} us")
    stream_read = stream_ceiling([int(head["launch_bytes"]), 512 << 20])
    cpu = cpu_extra = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.layout, args.query_tokens)
        if extra is not None:
            cpu_extra = cpu_baseline(args.extra_workload, args.layout, args.query_tokens)

    config, roofline = describe(head, args, args.layout)
    line = {
        "metric": METRIC, "value": round(head["worker_steps"], 3), "unit": "worker-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": head["wl"].kv_dtype, "data": "synthetic",
        "config": config, "spread": head["spread"], "roofline": roofline,
        "stream_read": stream_read, "cpu_baseline": cpu,
    }
    if extra is not None:
        xc, xr = describe(extra, args, args.layout)
        line[extra["wl"].name] = {
            "value": round(extra["worker_steps"], 3), "unit": "worker-steps/s",
            "ms_per_step": round(extra["ms_step"], 5), "spread": extra["spread"],
            "config": xc, "roofline": xr, "cpu_baseline": cpu_extra,
        }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
