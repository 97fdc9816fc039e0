#!/usr/bin/env python3
"""Benchmark of the Hogwild! concurrent-attention decode step on one MI355X.

A step is one decode step of every worker over every layer the workload times
(for w8_32k each layer first appends one new token per worker). Inputs are
seeded synthetic tensors already resident in HBM when the timed region starts.
With --query-tokens K > 1 every worker queries K tokens per step together
(hw_concurrent_decode_tokens: a paragraph header's tokens, causal), over the
same cache.

Prints ONE JSON line: worker-steps/s (value), the step's ideal-bytes GB/s,
a roofline object for the dominant kernel (concurrent_decode: algorithmic
bytes per launch / its average duration, from start/stop HIP events that the
kernel's own dispatch records on its stream during a timed pass), the measured
streaming-read ceiling of the same GPU (a plain 16-byte streaming-read kernel
at the decode launch's byte count and at 512 MiB, fresh memory each launch)
and the fp64 oracle's CPU rate on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "concurrent-attn decode worker-steps/s and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "shared_kv_cache_amd", "csrc", "hw_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="w4_16k",
                    choices=["tiny_fp32", "w2_4k", "w4_16k", "w8_32k", "w4_128k_sinks"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB copy kernel (counter calibration)")
    ap.add_argument("--splits", type=int, default=0, help="force KV partitions per head")
    ap.add_argument("--layout", default="combined",
                    choices=["combined", "stepwise", "contiguous", "nosync"],
                    help="cache layout the views follow (combined: the method's own)")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer pools to rotate through (0: the workload's own count; 1 keeps one "
                         "layer's K/V resident in the last-level cache)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the whole step captured as one HIP graph (workloads "
                         "whose views do not change between steps)")
    ap.add_argument("--query-tokens", type=int, default=1,
                    help="query tokens per worker and step (several: one causal decode of all)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the concurrent-"
              "attention step here is single-GPU by design", file=sys.stderr)
        return 2

    if args.query_tokens < 1:
        print("--query-tokens must be at least 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from shared_kv_cache_amd import hogwild as H
    from shared_kv_cache_amd import workloads as W

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    total_steps = args.warmup + 2 * args.steps + 1
    grows = args.workload == "w8_32k"
    extra = {"n_layers": args.layers} if args.layers > 0 else {}
    wl = W.make(args.workload, steps=total_steps if grows else 0, **extra)
    n, hq, hkv, d, L = wl.n_workers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_layers
    kv_dt = torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32
    elem = 2 if wl.kv_dtype == "bf16" else 4

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x torch.mul(src, 1.0, out=dst), 1 GiB read + 1 GiB written each")

    t0 = time.time()
    cache = H.HogwildCache(
        n_layers=L, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, page_size=wl.page_size,
        n_pages=wl.n_pages, max_blocks=len(wl.blocks()) + 1, max_workers=n,
        max_position=wl.max_position, kv_dtype=wl.kv_dtype, page_seed=wl.page_seed,
        rope_theta=wl.theta, max_splits=512 if args.splits > 256 else 0,
        max_query_tokens=args.query_tokens, device="cuda:0")
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
    kq = args.query_tokens
    n_q_steps = total_steps if grows and kq == 1 else 1

    def q_host(layer, s):
        return wl.q(layer, s) if kq == 1 else wl.q_tokens(layer, kq)

    q_dev = [[torch.from_numpy(q_host(layer, s if grows else 0)).to(dev) for s in range(n_q_steps)]
             for layer in range(L)]
    step_kv = None
    if grows:   # one new token per worker per layer per step, pre-staged in HBM
        step_kv = [[tuple(torch.from_numpy(x).to(dev).to(kv_dt) for x in wl.step_kv(layer, s + 1))
                    for s in range(total_steps)] for layer in range(L)]
    outs = [torch.empty((n, kq, hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    lses = [torch.empty((n, kq, hq), dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s: {wl.name}, {L} layers, T={wl.total_tokens()}")

    stream = torch.cuda.current_stream(dev).cuda_stream
    state = {"step": 0}

    def step():
        s = state["step"]
        for layer in range(L):
            if grows:
                k, v = step_kv[layer][s]
                H.hw_append_kv(cache.ctx, layer, wl.inprogress, [1] * n, k.data_ptr(),
                               v.data_ptr(), stream)
            q = q_dev[layer][s if n_q_steps > 1 else 0]
            if kq == 1:
                H.hw_concurrent_decode(cache.ctx, layer, q.data_ptr(), outs[layer].data_ptr(),
                                       lses[layer].data_ptr(), stream)
            else:
                H.hw_concurrent_decode_tokens(cache.ctx, layer, kq, q.data_ptr(),
                                              outs[layer].data_ptr(), lses[layer].data_ptr(), stream)
        state["step"] = s + 1

    def tokens_now():
        return sum(H.hw_block_info(cache.ctx, b, 0)[0] for b in blocks)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        if grows:
            print("--graph needs a workload whose views stay the same between steps", file=sys.stderr)
            return 2
        # The tables of the views are uploaded by the warm-up steps; the captured step holds
        # only the decode and merge launches of every layer.
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            stream = side.cuda_stream
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            stream = torch.cuda.current_stream(dev).cuda_stream
            step()
        stream = torch.cuda.current_stream(dev).cuda_stream
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    # Timed region 1: headline wall clock, no instrumentation.
    t_tok0 = tokens_now()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    t_tok1 = tokens_now()
    log(f"timed: {args.steps} steps in {ms_total:.3f} ms")

    # Timed region 2: the same steps, the decode kernels recording start/stop events.
    H.hw_debug_kernel_events(cache.ctx, args.steps * L)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dec_ms = H.hw_debug_kernel_elapsed(cache.ctx)
    H.hw_debug_kernel_events(cache.ctx, 0)
    res = H.hw_debug_resolve(cache.ctx, 0, n)
    # the resolver reports the one-token choice; several tokens per worker use more row
    # blocks and so fewer partitions
    n_splits = res["n_splits"] if kq == 1 else None

    # Algorithmic bytes: every K and V byte of the union of the views once per layer,
    # plus q read and out / lse written.
    avg_tokens = 0.5 * (t_tok0 + t_tok1) if grows else float(wl.total_tokens())
    kv_bytes = avg_tokens * hkv * d * 2 * elem
    io_bytes = n * kq * (hq * d * 4 * 2 + hq * 4)
    launch_bytes = kv_bytes + io_bytes
    append_bytes = (n * hkv * d * elem * 2 * 2) if grows else 0   # read + write new K and V
    step_bytes = L * (launch_bytes + append_bytes)
    ms_step = ms_total / args.steps
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9
    dec_avg = float(np.mean(dec_ms))
    achieved = launch_bytes / (dec_avg * 1e-3) / 1e9
    worker_steps = n * args.steps / (ms_total * 1e-3)

    stream_read = stream_ceiling(torch, H, dev, [int(launch_bytes), 512 << 20])
    cache.close()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, args.layout, kq)
    # the committed counters were taken on the default configuration of each workload
    default_cfg = (kq == 1 and args.layout == "combined" and not args.splits and not args.layers
                   and not args.graph)
    traffic = read_traffic(wl.name) if default_cfg else None

    line = {
        "metric": METRIC, "value": round(worker_steps, 3), "unit": "worker-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.kv_dtype, "data": "synthetic",
        "config": {
            "workload": wl.name, "layout": args.layout, "workers": n, "q_heads": hq,
            "kv_heads": hkv, "head_dim": d,
            "layers": L, "tokens_per_layer": round(avg_tokens, 1), "kv_dtype": wl.kv_dtype,
            "page_size": wl.page_size, "splits_per_head": n_splits,
            "step_ideal_bytes": int(step_bytes), "step_GBps": round(step_gbps, 1),
            "step_frac_of_hbm_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
            "decode_kernel_us": round(dec_avg * 1e3, 3),
            "appends_per_step": L if grows else 0, "query_tokens": kq, "hip_graph": graph is not None,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "stream_read": stream_read,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def stream_ceiling(torch, H, dev, sizes, reps=10):
    """Streaming-read ceiling: the library's plain read probe (16-byte streaming loads,
    every byte read once) over fresh windows of a 1 GiB buffer, so that no launch re-reads
    what the 256 MB last-level cache may still hold; median of `reps` launches timed by
    events of the kernel's own dispatch, best of two grid sizes."""
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


def cpu_baseline(wl, target_s: float, layout: str = "combined", query_tokens: int = 1):
    """The fp64 oracle, as it stands, on the host cores: whole layers of the workload
    (all workers, all query heads) until about target_s seconds have passed, with numpy's
    BLAS on every core this process may use; then one layer on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import hogwild_oracle as O

    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass

    def layer_inputs(layer):
        blocks = {b: tuple(x.astype(np.float64) for x in wl.kv(layer, b)) for b in wl.blocks()}
        q = wl.q(layer) if query_tokens == 1 else wl.q_tokens(layer, query_tokens)
        return blocks, q.astype(np.float64)

    done, t_sum = 0, 0.0
    with threadpool_limits(limits=threads):
        for layer in range(wl.n_layers):
            blocks, q = layer_inputs(layer)
            t0 = time.perf_counter()
            O.concurrent_attention(q, blocks, wl.views(layout), theta=wl.theta)
            t_sum += time.perf_counter() - t0
            done += 1
            if t_sum >= target_s:
                break
    with threadpool_limits(limits=1):
        blocks, q = layer_inputs(0)
        t0 = time.perf_counter()
        O.concurrent_attention(q, blocks, wl.views(layout), theta=wl.theta)
        one = time.perf_counter() - t0
    per_layer = t_sum / done
    rate = wl.n_workers / (per_layer * wl.n_layers)
    log(f"cpu oracle: {done} layers in {t_sum:.2f}s on {threads} threads -> {rate:.4f} "
        f"worker-steps/s; one layer on 1 thread {one:.2f}s")
    return {"value": round(rate, 5), "unit": "worker-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {wl.n_layers} layers at step 0, all {wl.n_workers} workers "
                      f"({query_tokens} query token(s) each) and "
                      f"{wl.n_q_heads} query heads; fp64 numpy oracle, BLAS on {threads} threads; "
                      f"rate = workers / (mean seconds per layer x {wl.n_layers} layers)",
            "cpu_model": model, "single_thread_s_per_layer": round(one, 3)}


if __name__ == "__main__":
    sys.exit(main())
