"""Benchmark of RocketKV's hot path on one MI355X.

Workload (default): the Llama3.1-8B-shaped layer at 128K context, bf16 (32 query / 8 KV heads,
head dim 128, batch 1; SnapKV++ window 32, pooling kernel 63, keep 16384; decode page size 4,
top 32 of 128 channels, top-k in {128, 512, 2048}, 256 decode steps each). To keep the
compressed state from being served by the 256 MB Infinity Cache, the layer is replicated as R
independently drawn layers (default 8, 640 MiB of compressed K/V + summaries) and consecutive
decode steps rotate through them, as a multi-layer model would.

One bench step = the whole hot path over that input: SnapKV++ eviction of every replica, page
summaries of every replica, then all decode steps (channel selection + approximate page scores,
page top-k, sparse attention: one fused kernel per step) for each top-k. Inputs are drawn on the
GPU before timing; each stage is captured once as a HIP graph and replayed, all on one stream.

value = mean fused decode-step latency (us) over the timed steps and top-k budgets; the JSON line
also carries per-top-k latency and GB/s, the dominant kernel's roofline, and, outside the timed
region: the per-stage split (the same steps as three separate calls), the multi-turn step over
the full 131072-token caches, a growing cache, selection quality, the other workloads (2K fp32,
32K, batch 16 at 32K, the 80-layer 70B-shaped stack at 256K, one 70B-shaped layer's eviction)
and the CPU oracle's time on bounded samples of every workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc-k_decode_step-llama8b-L131072-bf16.json")
COPY_CALIBRATION_BYTES = 256 << 20
DOMINANT = "k_decode_step"


def kernel_sources_digest() -> str:
    """sha256 over the HIP sources and headers of the library (the counters' validity key)."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "sparse_kv_cache_snapkv_amd", "csrc"), os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".hpp", ".h", ".cpp")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def summarize_pmc(fetch_csv: str, write_csv: str, out_json: str, kernel: str = DOMINANT) -> None:
    """Per-launch HBM traffic of a kernel (by default the dominant one) from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads
    for the plain 256 MiB device copy the run starts with (known bytes / counted bytes)."""
    import csv

    def dispatches(path, counter):
        rows = []
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return sorted(rows)

    out = dict(sources_sha256=kernel_sources_digest(), kernel=kernel,
               copy_bytes=COPY_CALIBRATION_BYTES)
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = dispatches(path, counter)
        # the calibration copy is the run's first copy kernel (inputs are drawn after it)
        copy = next(v for _, name, v in rows if "copy" in name)
        factor = COPY_CALIBRATION_BYTES / (copy * 1024.0)
        dom = [v for _, name, v in rows if kernel in name]
        out[counter] = dict(copy_kib=copy, factor=factor, launches=len(dom),
                            mean_kib_per_launch=sum(dom) / len(dom),
                            scaled_bytes_per_launch=sum(dom) / len(dom) * 1024.0 * factor)
    out["traffic_bytes_per_launch"] = (out["FETCH_SIZE"]["scaled_bytes_per_launch"]
                                       + out["WRITE_SIZE"]["scaled_bytes_per_launch"])
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def measured_traffic():
    """Scaled HBM bytes per launch of the dominant kernel, if taken on the current sources."""
    try:
        with open(PMC_SUMMARY) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    if pmc.get("sources_sha256") != kernel_sources_digest():
        return None
    return int(pmc["traffic_bytes_per_launch"])


def algorithmic_bytes(w, topk: int) -> dict:
    """Bytes the method must move per decode step and per stage launch (one layer)."""
    e = w.elem_bytes
    B, Hq, Hkv, D, P, r = w.B, w.Hq, w.Hkv, w.D, w.P, w.r
    n_pages = min(topk // w.page_size, P)
    k_tok = n_pages * w.page_size
    approx = B * Hkv * r * P * e + B * Hq * D * e + B * Hkv * P * 4
    topk_b = B * Hkv * P * 4 + B * Hkv * n_pages * 4
    attend = 2 * B * Hkv * k_tok * D * e + 2 * B * Hq * D * e + B * Hkv * n_pages * 4
    step = Hkv * e * (r * P + 2 * k_tok * D) * B + 2 * B * Hq * D * e + B * Hkv * n_pages * 4
    summaries = B * Hkv * w.Lc * D * e + 2 * B * Hkv * P * D * e
    evict = (B * Hkv * w.L * D * e + B * w.Hq * w.W * D * e + 4 * B * Hkv * w.keep * D * e
             + B * Hkv * w.keep * 4)
    return dict(step=step, approx=approx, topk=topk_b, attend=attend, summaries=summaries,
                evict=evict)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def gbps(nbytes, us):
    return round(nbytes / (us * 1e-6) / 1e9, 1)


def replay_us(torch, graph, reps: int) -> float:
    """Median over `reps` replays of one captured graph, in microseconds per replay."""
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def capture(torch, fn):
    """Runs fn once (eagerly, on the current stream, then synchronises) and captures it."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def decode_rows(rkv, torch, w, k_c, v_c, kmin, kmax, R, nsteps, reps, q_dec=None, rows=None,
                full_k=None, full_v=None):
    """Fused decode steps of workload w over R replicas (replica r is batch slice r*B .. r*B+B-1
    of the caches; consecutive steps rotate through them), for every top-k: graph replay time per
    step, algorithmic bytes, GB/s and the HBM fraction. With rows (the SnapKV++ kept indices) and
    the full caches, the multi-turn step over the view of the full cache is timed instead."""
    import math
    B = w.B
    scale = 1.0 / math.sqrt(w.D)
    if q_dec is None:
        from workloads import generate as gen
        q_dec = gen.device_decode_queries(w, 0, nsteps, torch.device("cuda:0"))
    out = torch.empty((nsteps,) + tuple(q_dec.shape[1:]), dtype=q_dec.dtype, device="cuda:0")
    res = {}
    for tk in w.topk:
        n_pages = min(tk // w.page_size, w.P)
        pages = torch.empty((B, w.Hkv, n_pages), dtype=torch.int32, device="cuda:0")
        ws = rkv.rkv_hybrid_decode_workspace(q_dec[0], w.Hkv, w.Lc, w.page_size, n_pages)

        def run():
            for s in range(nsteps):
                r = s % R
                sl = slice(r * B, (r + 1) * B)
                if rows is None:
                    rkv.rkv_hybrid_decode_step(q_dec[s], kmin[sl], kmax[sl], k_c[sl], v_c[sl],
                                               w.page_size, w.r, n_pages, scale, page_idx=pages,
                                               out=out[s], workspace=ws)
                else:
                    rkv.rkv_hybrid_decode_step_indexed(q_dec[s], kmin[sl], kmax[sl], full_k[r],
                                                       full_v[r], rows[sl], w.page_size, w.r,
                                                       n_pages, scale, page_idx=pages, out=out[s],
                                                       workspace=ws)

        g = capture(torch, run)
        us = replay_us(torch, g, reps) / nsteps
        ab = algorithmic_bytes(w, tk)["step"]
        res[str(tk)] = dict(us_per_step=round(us, 3), algorithmic_bytes=ab, GBps=gbps(ab, us),
                            hbm_frac=round(ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                            status=rkv.decode_workspace_status(ws))
        del g, ws, pages
    return res


def evict_70b_layer(rkv, torch, reps: int = 3) -> dict:
    """SnapKV++ eviction of one layer of the 70B-shaped workload (64/8 heads, D 128, context
    262144, window 64, keep 32768): the shape where the window passes are bound by MFMA and the
    exponentials rather than by HBM. Events around `reps` calls after one warm-up call."""
    from workloads import configs, generate as gen
    import math
    w = configs.LLAMA70B_256K_80L
    dev = torch.device("cuda:0")
    p = gen.device_prompt_layer(w, 0, dev)
    B, Hq, Hkv, D, L, W, keep = w.B, w.Hq, w.Hkv, w.D, w.L, w.W, w.keep
    kept = torch.empty((B, Hkv, keep), dtype=torch.int32, device=dev)
    kc = torch.empty((B, Hkv, keep, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    ws = torch.empty(rkv.snapkvpp_workspace_bytes(B, Hq, Hkv, L, D, W, keep, 1),
                     dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)

    def run():
        rkv.rkv_snapkvpp_evict(p["q_win"], p["k"], p["v"], keep, w.pool_kernel, "avg", scale,
                               kept_idx=kept, k_out=kc, v_out=vc, workspace=ws)

    torch.cuda.synchronize()
    run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    flops = 4 * B * Hq * W * L * D  # the two window passes' QK^T
    nb = algorithmic_bytes(w, w.topk[0])["evict"]
    del p, kept, kc, vc, ws
    return dict(workload=w.name, us_per_layer=round(us, 1), mfma_flops=flops,
                mfma_TFLOPs=round(flops / (us * 1e-6) / 1e12, 1),
                mfma_frac=round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                algorithmic_bytes=nb, GBps=gbps(nb, us))


def batch16_decode(rkv, torch, replicas: int, reps: int) -> dict:
    """The batch-16 workload (16 sequences at 32K, 8B-shaped, top-k 256): R independently drawn
    batches, each evicted with SnapKV++ and summarised, then fused decode steps rotating through
    them (4 x 288 MiB of compressed state, above the Infinity Cache): tokens x heads per second,
    GB/s and the HBM fraction."""
    from workloads import configs, runs
    w = configs.LLAMA8B_32K_B16
    st = runs.compressed_stack(rkv, w, replicas)
    kmin, kmax = rkv.rkv_build_page_summaries(st["k_c"], w.page_size)
    res = decode_rows(rkv, torch, w, st["k_c"], st["v_c"], kmin, kmax, replicas, w.steps, reps)
    for tk, row in res.items():
        row["tokens_heads_per_s"] = round(w.B * w.Hq / (row["us_per_step"] * 1e-6), 1)
    ok = st["needles_ok"]
    del st, kmin, kmax
    return dict(workload=w.name, batch=w.B, replicas=replicas, decode_steps=w.steps,
                needles_kept=ok, per_topk=res)


def layers80_decode(rkv, torch, reps: int) -> dict:
    """The 70B-shaped workload: 80 independently drawn layers at 256K, each evicted with SnapKV++
    (keep 32768) and summarised; one decode step of attention for all 80 layers is one fused
    launch over 640 heads (the layers are independent, so they fold into the batch), 16 steps."""
    from workloads import configs, runs
    w = configs.LLAMA70B_256K_80L
    L = w.layers
    st = runs.compressed_stack(rkv, w, L,
                               on_layer=lambda i: progress(f"layers80: layer {i} evicted")
                               if i % 10 == 9 else None)
    kmin, kmax = rkv.rkv_build_page_summaries(st["k_c"], w.page_size)
    wl = w.replace(B=L * w.B)
    res = decode_rows(rkv, torch, wl, st["k_c"], st["v_c"], kmin, kmax, 1, w.steps, reps)
    ok = st["needles_ok"]
    del st, kmin, kmax
    return dict(workload=w.name, layers=L, heads_per_launch=wl.B * w.Hkv, decode_steps=w.steps,
                needles_kept=ok, per_topk=res)


def small_decode(rkv, torch, w, reps: int) -> dict:
    """Fused decode latency of a one-layer workload (R = 1; its compressed state is small)."""
    from workloads import runs
    st = runs.compressed_stack(rkv, w, 1)
    kmin, kmax = rkv.rkv_build_page_summaries(st["k_c"], w.page_size)
    res = decode_rows(rkv, torch, w, st["k_c"], st["v_c"], kmin, kmax, 1, w.steps, reps)
    del st, kmin, kmax
    return dict(workload=w.name, decode_steps=w.steps, per_topk=res)


def oracle_config(w, heads, steps: int, one_thread: bool) -> dict:
    """The oracle, as it stands, on a sample of one workload: SnapKV++ eviction and `steps` decode
    steps per top-k for each sampled (layer, b, KV head), scaled to the whole step (x heads per
    layer; with several layers, x layers, labelled extrapolated)."""
    import numpy as np
    from oracle import rocketkv as O
    from workloads import generate as gen
    scale = 1.0 / math.sqrt(w.D)

    def run():
        ev, dec = [], {tk: [] for tk in w.topk}
        for (layer, b, h) in heads:
            hd = gen.prompt_head(w, layer, b, h)
            q_win = O.widen(gen.to_storage(hd["q_win"], w.dtype))
            k = O.widen(gen.to_storage(hd["k"], w.dtype))
            v = O.widen(gen.to_storage(hd["v"], w.dtype))
            t0 = time.perf_counter()
            kept, _, _ = O.snapkvpp_head(q_win, k, w.keep, w.pool_kernel, scale)
            ev.append(time.perf_counter() - t0)
            kc, vc = k[kept], v[kept]
            kmin, kmax = O.page_summaries(kc, w.page_size)
            rng = np.random.default_rng(layer * 1000 + b * 10 + h)
            for tk in w.topk:
                n_pages = min(tk // w.page_size, w.P)
                t0 = time.perf_counter()
                for _ in range(steps):
                    qg = rng.standard_normal((w.G, w.D))
                    chans, qbar = O.select_channels(qg, w.r)
                    sc = O.approx_page_scores(qbar, chans, kmin, kmax)
                    pages = O.select_pages(sc, n_pages)
                    O.sparse_attention(qg, kc, vc, O.page_tokens(pages, w.page_size, w.Lc), scale)
                dec[tk].append((time.perf_counter() - t0) / steps)
        per_layer_heads = w.B * w.Hkv
        mult = per_layer_heads * w.layers
        decode_us = {str(tk): round(sum(v) / len(v) * 1e6 * mult, 1) for tk, v in dec.items()}
        return dict(evict_ms=round(sum(ev) / len(ev) * 1e3 * mult, 1), decode_step_us=decode_us)

    res = run()
    if one_thread:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = run()
        res["one_thread"] = one
    res["sample"] = (f"(layer, b, KV head) {list(heads)}: eviction once and {steps} decode steps per "
                     f"top-k each; scaled x{w.B * w.Hkv} heads per layer"
                     + (f" x{w.layers} layers (extrapolated)" if w.layers > 1 else ""))
    return res


def cpu_baseline(w_main, sample_steps: int) -> dict:
    """The oracle on the host cores, on bounded samples of every workload; the headline figure
    is the 128K layer's decode step (mean over its top-k budgets)."""
    from workloads import configs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    per_config = {}
    plan = [(configs.TINY_FP32, [(0, 0, 0), (0, 0, 1)], 8, True),
            (configs.LLAMA8B_32K, [(0, 0, 0)], 8, True),
            (w_main, [(0, 0, 0)], sample_steps, False),
            (configs.LLAMA8B_32K_B16, [(0, 0, 0)], 8, False),
            (configs.LLAMA70B_256K_80L, [(0, 0, 0), (79, 0, 0)], 4, False)]
    for w, heads, steps, one in plan:
        per_config[w.name] = oracle_config(w, heads, steps, one)
    main = per_config[w_main.name]["decode_step_us"]
    value = sum(main.values()) / len(main)
    return dict(value=round(value, 1), unit="us per decode step", cores=blas_threads,
                cores_meaning="BLAS threads the oracle's matrix products ran on",
                host_cores_available=len(os.sched_getaffinity(0)), kind="oracle",
                sample=per_config[w_main.name]["sample"] + "; mean over top-k",
                per_config=per_config)


def calibration_copy(torch, dev) -> None:
    """A plain device copy of COPY_CALIBRATION_BYTES, the counters' scale."""
    src = torch.ones(COPY_CALIBRATION_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _other_workloads():
    from workloads import configs
    return {
        "tiny": lambda rkv, torch, reps: small_decode(rkv, torch, configs.TINY_FP32, reps),
        "llama8b_32k": lambda rkv, torch, reps: small_decode(rkv, torch, configs.LLAMA8B_32K, reps),
        "batch16": lambda rkv, torch, reps: batch16_decode(rkv, torch, 4, reps),
        "layers80": lambda rkv, torch, reps: layers80_decode(rkv, torch, reps),
        "evict_70b_layer": lambda rkv, torch, reps: evict_70b_layer(rkv, torch),
    }


OTHER_WORKLOADS = _other_workloads()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b-L131072-bf16")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--cpu-sample-steps", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the timed pass and the headline fields (profiling runs)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="start with a plain 256 MiB device copy (the counters' scale)")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="write the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--pmc-kernel", default=DOMINANT,
                    help="kernel-name substring whose launches --pmc-summary averages")
    ap.add_argument("--only", choices=sorted(OTHER_WORKLOADS),
                    help="run only this other workload's section and print its JSON (profiling)")
    args = ap.parse_args()
    if args.pmc_summary:
        summarize_pmc(*args.pmc_summary, kernel=args.pmc_kernel)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the RocketKV path here runs on a single MI355X "
              "(no sharding or collectives are built); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import sparse_kv_cache_snapkv_amd as rkv
    from workloads import configs, generate as gen

    w = configs.by_name(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only:
        if args.pmc_calibration:
            calibration_copy(torch, dev)
        print(json.dumps({args.only: OTHER_WORKLOADS[args.only](rkv, torch, 5)}), flush=True)
        return 0
    R = args.replicas
    nsteps = args.decode_steps or w.steps
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dcode = 1 if w.dtype == "bf16" else 0
    B, Hq, Hkv, D, Lc, P = w.B, w.Hq, w.Hkv, w.D, w.Lc, w.P
    scale = 1.0 / math.sqrt(D)
    reps = 5

    if args.pmc_calibration:
        calibration_copy(torch, dev)

    # ---- inputs resident in HBM, outputs and workspaces preallocated. Everything runs on the
    # current (default) stream: each stage is run once eagerly, then captured as a HIP graph.
    prompts = [gen.device_prompt_layer(w, layer, dev) for layer in range(R)]
    for p in prompts:
        del p["needle_dir"]
    q_dec = gen.device_decode_queries(w, 0, nsteps, dev)
    kept = torch.empty((R, B, Hkv, Lc), dtype=torch.int32, device=dev)
    k_c = torch.empty((R, B, Hkv, Lc, D), dtype=dt, device=dev)
    v_c = torch.empty_like(k_c)
    kmin = torch.empty((R, B, Hkv, D, P), dtype=dt, device=dev)
    kmax = torch.empty_like(kmin)
    ev_ws = torch.empty(max(1, rkv.snapkvpp_workspace_bytes(B, Hq, Hkv, w.L, D, w.W, w.keep, dcode)),
                        dtype=torch.uint8, device=dev)
    n_pages = {tk: min(tk // w.page_size, P) for tk in w.topk}
    pages = {tk: torch.empty((B, Hkv, n_pages[tk]), dtype=torch.int32, device=dev) for tk in w.topk}
    dec_ws = {tk: rkv.rkv_hybrid_decode_workspace(q_dec[0], Hkv, Lc, w.page_size, n_pages[tk])
              for tk in w.topk}
    out = torch.empty((nsteps, B, Hq, D), dtype=dt, device=dev)

    def evict_all():
        for r in range(R):
            p = prompts[r]
            rkv.rkv_snapkvpp_evict(p["q_win"], p["k"], p["v"], w.keep, w.pool_kernel, "avg", scale,
                                   kept_idx=kept[r], k_out=k_c[r], v_out=v_c[r], workspace=ev_ws)

    def summarize_all():
        for r in range(R):
            rkv.rkv_build_page_summaries(k_c[r], w.page_size, kmin_t=kmin[r], kmax_t=kmax[r])

    def decode_all(tk):
        # one fused kernel per decode step; consecutive steps rotate through the layer replicas
        for s in range(nsteps):
            r = s % R
            rkv.rkv_hybrid_decode_step(q_dec[s], kmin[r], kmax[r], k_c[r], v_c[r], w.page_size,
                                       w.r, n_pages[tk], scale, page_idx=pages[tk], out=out[s],
                                       workspace=dec_ws[tk])

    stages = [("evict", evict_all), ("summaries", summarize_all)] + \
             [(f"decode@{tk}", (lambda tk=tk: decode_all(tk))) for tk in w.topk]
    graphs = {name: capture(torch, fn) for name, fn in stages}

    def one_pass(ev=None):
        for name, _ in stages:
            if ev is not None:
                ev[name][0].record()
            graphs[name].replay()
            if ev is not None:
                ev[name][1].record()

    progress("warm-up")
    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    progress("timed passes")

    # ---- timed region: K whole passes (eviction, summaries, every decode step of every top-k)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    wall0 = time.perf_counter()
    stage_ms = {name: 0.0 for name, _ in stages}
    for _ in range(args.steps):
        ev = {name: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for name, _ in stages}
        one_pass(ev)
        torch.cuda.synchronize()
        for name in stage_ms:
            stage_ms[name] += ev[name][0].elapsed_time(ev[name][1]) / args.steps
    t_end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3
    pass_ms = t_start.elapsed_time(t_end) / args.steps
    status = {tk: rkv.decode_workspace_status(dec_ws[tk]) for tk in w.topk}

    per_topk, stages_out = {}, {}
    for name, ms in stage_ms.items():
        kind, _, tk = name.partition("@")
        ab = algorithmic_bytes(w, int(tk) if tk else w.topk[0])
        if kind == "decode":
            us = ms * 1e3 / nsteps
            per_topk[tk] = dict(us_per_step=round(us, 3), algorithmic_bytes=ab["step"],
                                GBps=gbps(ab["step"], us),
                                hbm_frac=round(ab["step"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4))
        else:
            nb = ab[kind] * R
            stages_out[name] = dict(us_total=round(ms * 1e3, 2), us_per_layer=round(ms * 1e3 / R, 2),
                                    algorithmic_bytes=nb, GBps=gbps(nb, ms * 1e3))

    # dominant kernel: the fused decode-step kernel, one launch per step, over all of its launches
    # in the timed region (every top-k); its launch duration is the graph-replay time per step
    dom_us = sum(per_topk[str(tk)]["us_per_step"] for tk in w.topk) / len(w.topk)
    bytes_per_launch = sum(algorithmic_bytes(w, tk)["step"] for tk in w.topk) / len(w.topk)
    achieved = bytes_per_launch / (dom_us * 1e-6) / 1e9
    roofline = dict(kernel="k_decode_step (fused decode step), mean over top-k "
                           + "/".join(str(t) for t in w.topk),
                    bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=measured_traffic(),
                    algorithmic_bytes_per_launch=int(bytes_per_launch),
                    avg_launch_us=round(dom_us, 3))
    value = sum(v["us_per_step"] for v in per_topk.values()) / len(per_topk)
    line = dict(
        metric="decode-step sparse attention latency (us) + achieved HBM GB/s, 8B shape @128K",
        value=round(value, 3), unit="us", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(pass_ms, 3), higher_is_better=False, scaling="weak", vs_baseline=None,
        dtype=w.dtype, data="synthetic",
        config=dict(workload=w.name, batch=B, query_heads=Hq, kv_heads=Hkv, head_dim=D,
                    context=w.L, window=w.W, pool_kernel=w.pool_kernel, keep=w.keep,
                    page_size=w.page_size, channels=w.r, topk=list(w.topk),
                    decode_steps=nsteps, replicas=R),
        per_topk=per_topk, stages=stages_out, roofline=roofline, sync_status=status,
        wall_ms_timed=round(wall_ms, 1))

    if not args.no_extra:
        extra(rkv, torch, gen, w, line, prompts, kept, k_c, v_c, kmin, kmax, q_dec, out, nsteps, R,
              reps)
    del graphs
    if not args.no_cpu_baseline:
        progress("oracle on the host")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_steps)
    print(json.dumps(line), flush=True)
    return 0


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def extra(rkv, torch, gen, w, line, prompts, kept, k_c, v_c, kmin, kmax, q_dec, out, nsteps, R,
          reps):
    """Everything outside the timed region, added to the JSON line."""
    from workloads import configs
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, Lc, P = w.B, w.Hq, w.Hkv, w.D, w.Lc, w.P
    scale = 1.0 / math.sqrt(D)
    dt = k_c.dtype

    progress("three-call split")
    # the same decode steps as three separate calls, stage by stage (the per-stage split)
    scores = torch.empty((B, Hkv, P), dtype=torch.float32, device=dev)
    split = {}
    for tk in w.topk:
        n_pages = min(tk // w.page_size, P)
        pages = torch.empty((B, Hkv, n_pages), dtype=torch.int32, device=dev)
        att_ws = torch.empty(max(1, rkv.sparse_attend_workspace_bytes(
            B, Hq, Hkv, D, w.page_size, n_pages, 1 if dt == torch.bfloat16 else 0)),
            dtype=torch.uint8, device=dev)

        def approx_all():
            for s in range(nsteps):
                r = s % R
                rkv.rkv_hybrid_approx_scores(q_dec[s], kmin[r], kmax[r], w.r, page_scores=scores)

        def topk_all():
            for s in range(nsteps):
                rkv.rkv_topk_select(scores, n_pages, idx_out=pages)

        def attend_all():
            for s in range(nsteps):
                r = s % R
                rkv.rkv_sparse_attend_decode(q_dec[s], k_c[r], v_c[r], pages, w.page_size, scale,
                                             out=out[s], workspace=att_ws)

        ab = algorithmic_bytes(w, tk)
        us = {k: replay_us(torch, capture(torch, fn), reps) / nsteps
              for k, fn in (("approx", approx_all), ("topk", topk_all), ("attend", attend_all))}
        split[str(tk)] = dict(approx_us=round(us["approx"], 3), approx_bytes=ab["approx"],
                              topk_us=round(us["topk"], 3), topk_bytes=ab["topk"],
                              attend_us=round(us["attend"], 3), attend_bytes=ab["attend"],
                              sum_us=round(sum(us.values()), 3))
        line["per_topk"][str(tk)]["three_calls"] = split[str(tk)]
        del pages, att_ws

    progress("multi-turn step over the full caches")
    # RocketKV-MT: the step over the view of every replica's full 131072-token cache through
    # SnapKV++'s kept rows (summaries of the view built by the indexed call)
    kmin_mt = torch.empty_like(kmin)
    kmax_mt = torch.empty_like(kmax)
    for r in range(R):
        rkv.rkv_build_page_summaries_indexed(prompts[r]["k"], kept[r], w.page_size,
                                             kmin_t=kmin_mt[r], kmax_t=kmax_mt[r])
    torch.cuda.synchronize()
    same = bool(torch.equal(kmin_mt, kmin) and torch.equal(kmax_mt, kmax))
    full_k = [p["k"] for p in prompts]
    full_v = [p["v"] for p in prompts]
    mt = decode_rows(rkv, torch, w, None, None, kmin_mt.view(R * B, Hkv, D, P),
                     kmax_mt.view(R * B, Hkv, D, P), R, nsteps, reps, q_dec=q_dec,
                     rows=kept.view(R * B, Hkv, Lc), full_k=full_k, full_v=full_v)
    line["multi_turn"] = dict(workload=w.name + " (view of the full caches)", context=w.L,
                              summaries_equal_to_evicted=same, per_topk=mt)
    del kmin_mt, kmax_mt

    progress("growing cache")
    # a cache that grows during decoding (replica 0's compressed layer copied into caches of
    # capacity Lc + nsteps): one append per step, then the same appends each followed by the
    # fused step on the grown cache (smallest top-k)
    cap = Lc + nsteps
    kc_g = torch.zeros((B, Hkv, cap, D), dtype=dt, device=dev)
    vc_g = torch.zeros_like(kc_g)
    kc_g[:, :, :Lc] = k_c[0]
    vc_g[:, :, :Lc] = v_c[0]
    kmin_g, kmax_g = rkv.rkv_build_page_summaries_cap(kc_g, Lc, w.page_size)
    gg = torch.Generator(device=dev).manual_seed(1)
    k_new = torch.randn((nsteps, B, Hkv, D), device=dev, generator=gg).to(dt)
    v_new = torch.randn((nsteps, B, Hkv, D), device=dev, generator=gg).to(dt)
    tk_g = w.topk[0]
    n_g = min(tk_g // w.page_size, P)
    ws_g = rkv.rkv_hybrid_decode_workspace(q_dec[0], Hkv, cap, w.page_size, n_g)

    def append_all():
        for s in range(nsteps):
            rkv.rkv_kv_append(k_new[s], v_new[s], kc_g, vc_g, kmin_g, kmax_g, Lc + s, w.page_size)

    def grow_all():
        for s in range(nsteps):
            rkv.rkv_kv_append(k_new[s], v_new[s], kc_g, vc_g, kmin_g, kmax_g, Lc + s, w.page_size)
            rkv.rkv_hybrid_decode_step_cap(q_dec[s], kmin_g, kmax_g, kc_g, vc_g, Lc + s + 1,
                                           w.page_size, w.r, n_g, scale, out=out[s],
                                           workspace=ws_g)

    grow = {k: replay_us(torch, capture(torch, fn), reps) / nsteps
            for k, fn in (("append", append_all), ("append+step", grow_all))}
    line["growing_cache"] = dict(capacity=cap, appends=nsteps, append_us=round(grow["append"], 3),
                                 append_bytes=8 * B * Hkv * D * (2 if dt == torch.bfloat16 else 4),
                                 append_plus_step_us=round(grow["append+step"], 3),
                                 step_topk=tk_g, sync_status=rkv.decode_workspace_status(ws_g))
    del kc_g, vc_g, kmin_g, kmax_g, ws_g

    progress("selection quality")
    # selection quality against Exact-TopK (replica 0, the first decode steps): RocketKV's split
    # against QUEST-like and SparQ-like settings of the same approximation ratio (ps * D / r)
    from sparse_kv_cache_snapkv_amd import quality
    ratio = w.page_size * D // w.r
    settings = dict(hybrid=(w.page_size, w.r), quest_like=(ratio, D),
                    sparq_like=(1, max(1, D // ratio)))
    qsteps = 4
    sel_q = {name: {str(tk): dict(recall=0.0, mass=0.0, mass_exact=0.0) for tk in w.topk}
             for name in settings}
    for s in range(qsteps):
        ex = quality.exact_scores(q_dec[s], k_c[0])
        for name, (ps_q, r_q) in settings.items():
            for tk in w.topk:
                m = quality.selection_quality(q_dec[s], k_c[0], ps_q, r_q, tk, scale, exact=ex)
                for key in m:
                    sel_q[name][str(tk)][key] += m[key] / qsteps
    for name in sel_q:
        for tk in sel_q[name]:
            sel_q[name][tk] = {k: round(v, 4) for k, v in sel_q[name][tk].items()}
    sel_q["settings"] = {name: dict(page_size=ps_q, r=r_q) for name, (ps_q, r_q) in settings.items()}
    sel_q["decode_steps"] = qsteps
    line["selection_quality"] = sel_q

    progress("other workloads")
    # the other workloads: decode latency at 2K (fp32) and 32K, the batch-16 workload, the
    # 80-layer 70B-shaped stack, and one 70B-shaped layer's eviction
    torch.cuda.empty_cache()
    other = {}
    for name in ("tiny", "llama8b_32k", "batch16", "layers80", "evict_70b_layer"):
        progress(name)
        other[name] = OTHER_WORKLOADS[name](rkv, torch, reps)
        torch.cuda.empty_cache()
    line["other_workloads"] = other
    torch.cuda.empty_cache()


if __name__ == "__main__":
    sys.exit(main())
