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
GPU before timing; each stage is captured once as a HIP graph and replayed. The per-stage split
of a decode step is measured beside it by the same steps run as the three separate calls
(approximate scores, page top-k, sparse attention), each stage a graph of its own.

value = mean fused decode-step latency (us) over the timed steps and top-k budgets; the JSON line
also carries per-top-k latency and GB/s, the per-stage split, the dominant kernel's roofline,
and the CPU oracle's time on a bounded sample.
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


def summarize_pmc(fetch_csv: str, write_csv: str, out_json: str) -> None:
    """Per-launch HBM traffic of the dominant kernel from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads for the plain
    256 MiB device copy the run starts with (known bytes / counted bytes)."""
    import csv

    def dispatches(path, counter):
        rows = []
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return sorted(rows)

    out = dict(sources_sha256=kernel_sources_digest(), kernel=DOMINANT,
               copy_bytes=COPY_CALIBRATION_BYTES)
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = dispatches(path, counter)
        # the calibration copy is the run's first copy kernel (inputs are drawn after it)
        copy = next(v for _, name, v in rows if "copy" in name)
        factor = COPY_CALIBRATION_BYTES / (copy * 1024.0)
        dom = [v for _, name, v in rows if DOMINANT in name]
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


def evict_70b_layer(rkv, torch, reps: int = 3) -> dict:
    """SnapKV++ eviction of one layer of the 70B-shaped workload (64/8 heads, D 128, context
    262144, window 64, keep 32768): the shape where the window passes are bound by MFMA and the
    exponentials rather than by HBM. Default stream, inputs resident, events around `reps`
    calls after one warm-up call."""
    from workloads import configs, generate as gen
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
    nb = (B * Hkv * L * D * 2 + B * Hq * W * D * 2 + 4 * B * Hkv * keep * D * 2
          + B * Hkv * keep * 4)
    del p, kept, kc, vc, ws
    torch.cuda.empty_cache()
    return dict(workload=w.name, us_per_layer=round(us, 1), mfma_flops=flops,
                mfma_TFLOPs=round(flops / (us * 1e-6) / 1e12, 1),
                mfma_frac=round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                algorithmic_bytes=nb, GBps=round(nb / (us * 1e-6) / 1e9, 1))


def cpu_baseline(w, sample_steps: int):
    """The oracle, as it stands, on one KV head of the workload; scaled to us per decode step."""
    import numpy as np
    from oracle import rocketkv as O
    from workloads import generate as gen
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    hd = gen.prompt_head(w, 0, 0, 0)
    q_win = O.widen(gen.to_storage(hd["q_win"], w.dtype))
    k = O.widen(gen.to_storage(hd["k"], w.dtype))
    v = O.widen(gen.to_storage(hd["v"], w.dtype))
    scale = 1.0 / math.sqrt(w.D)
    t0 = time.perf_counter()
    kept, _, _ = O.snapkvpp_head(q_win, k, w.keep, w.pool_kernel, scale)
    t_evict = time.perf_counter() - t0
    kc, vc = k[kept], v[kept]
    kmin, kmax = O.page_summaries(kc, w.page_size)
    rng = np.random.default_rng(0)
    per_k = {}
    for tk in w.topk:
        n_pages = min(tk // w.page_size, w.P)
        t0 = time.perf_counter()
        for _ in range(sample_steps):
            qg = rng.standard_normal((w.G, w.D))
            chans, qbar = O.select_channels(qg, w.r)
            sc = O.approx_page_scores(qbar, chans, kmin, kmax)
            pages = O.select_pages(sc, n_pages)
            O.sparse_attention(qg, kc, vc, O.page_tokens(pages, w.page_size, w.Lc), scale)
        per_k[tk] = (time.perf_counter() - t0) / sample_steps * 1e6 * w.Hkv * w.B
    value = sum(per_k.values()) / len(per_k)
    return dict(value=round(value, 1), unit="us per decode step", cores=blas_threads,
                host_cores_available=cores, kind="oracle",
                sample=(f"1 of {w.B * w.Hkv} KV heads: SnapKV++ eviction once "
                        f"({t_evict:.2f} s) and {sample_steps} decode steps per top-k "
                        f"{list(w.topk)}, scaled x{w.B * w.Hkv} heads; mean over top-k"),
                per_topk_us={str(k): round(x, 1) for k, x in per_k.items()},
                evict_s_per_layer=round(t_evict * w.B * w.Hkv, 2))


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
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="start with a plain 256 MiB device copy (the counters' scale)")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="write the traffic summary of two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        summarize_pmc(*args.pmc_summary)
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
    R = args.replicas
    nsteps = args.decode_steps or w.steps
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dcode = 1 if w.dtype == "bf16" else 0
    B, Hq, Hkv, D, Lc, P, G = w.B, w.Hq, w.Hkv, w.D, w.Lc, w.P, w.G
    scale = 1.0 / math.sqrt(D)

    if args.pmc_calibration:
        src = torch.ones(COPY_CALIBRATION_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- inputs resident in HBM, outputs and workspaces preallocated
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
    scores = torch.empty((B, Hkv, P), dtype=torch.float32, device=dev)
    att_ws = {tk: torch.empty(max(1, rkv.sparse_attend_workspace_bytes(B, Hq, Hkv, D, w.page_size,
                                                                      n_pages[tk], dcode)),
                              dtype=torch.uint8, device=dev) for tk in w.topk}

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

    # the same decode steps as three separate calls, stage by stage (for the per-stage split)
    def approx_all():
        for s in range(nsteps):
            r = s % R
            rkv.rkv_hybrid_approx_scores(q_dec[s], kmin[r], kmax[r], w.r, page_scores=scores)

    def topk_all(tk):
        for s in range(nsteps):
            rkv.rkv_topk_select(scores, n_pages[tk], idx_out=pages[tk])

    def attend_all(tk):
        for s in range(nsteps):
            r = s % R
            rkv.rkv_sparse_attend_decode(q_dec[s], k_c[r], v_c[r], pages[tk], w.page_size,
                                         scale, out=out[s], workspace=att_ws[tk])

    # ---- capture each stage as a HIP graph (launch-bound loops replay without host overhead)
    stages = [("evict", evict_all), ("summaries", summarize_all)] + \
             [(f"decode@{tk}", (lambda tk=tk: decode_all(tk))) for tk in w.topk]
    split_stages = [("split_approx", approx_all)] + \
                   [(f"split_topk@{tk}", (lambda tk=tk: topk_all(tk))) for tk in w.topk] + \
                   [(f"split_attend@{tk}", (lambda tk=tk: attend_all(tk))) for tk in w.topk]
    side = torch.cuda.Stream()
    # inputs, summaries and workspaces (with their zero-fill) were made on the default stream: the
    # warm-up on the side stream may only start once they exist
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _, fn in stages + split_stages:
            fn()
    torch.cuda.synchronize()
    graphs = {}
    for name, fn in stages + split_stages:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g

    def one_pass(ev=None, which=stages):
        for name, _ in which:
            if ev is not None:
                ev[name][0].record()
            graphs[name].replay()
            if ev is not None:
                ev[name][1].record()

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()

    # ---- timed region: K whole passes
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

    # ---- outside the timed region: the same decode steps as three separate calls
    one_pass(which=split_stages)
    for _ in range(args.steps):
        ev = {name: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for name, _ in split_stages}
        one_pass(ev, which=split_stages)
        torch.cuda.synchronize()
        for name in ev:
            stage_ms[name] = stage_ms.get(name, 0.0) + ev[name][0].elapsed_time(ev[name][1]) / args.steps
    if any(status.values()):
        print(f"warning: a fused decode step reported a synchronisation timeout {status}",
              file=sys.stderr)

    # ---- outside the timed region: a cache that grows during decoding (replica 0's compressed
    # layer copied into caches of capacity Lc + nsteps): one append per step, then the same
    # appends each followed by the fused step on the grown cache (smallest top-k)
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
    ws_g = rkv.rkv_hybrid_decode_workspace(q_dec[0], Hkv, cap, w.page_size, n_pages[tk_g])

    def append_all():
        for s in range(nsteps):
            rkv.rkv_kv_append(k_new[s], v_new[s], kc_g, vc_g, kmin_g, kmax_g, Lc + s, w.page_size)

    def grow_all():
        for s in range(nsteps):
            rkv.rkv_kv_append(k_new[s], v_new[s], kc_g, vc_g, kmin_g, kmax_g, Lc + s, w.page_size)
            rkv.rkv_hybrid_decode_step_cap(q_dec[s], kmin_g, kmax_g, kc_g, vc_g, Lc + s + 1,
                                           w.page_size, w.r, n_pages[tk_g], scale, out=out[s],
                                           workspace=ws_g)

    grow_us = {}
    torch.cuda.synchronize()  # the grown caches and their workspace exist before the side stream
    for name, fn in (("append", append_all), ("append+step", grow_all)):
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(args.steps):
            g.replay()
        a1.record()
        torch.cuda.synchronize()
        grow_us[name] = a0.elapsed_time(a1) * 1e3 / (args.steps * nsteps)
    app_bytes = 8 * B * Hkv * D * w.elem_bytes  # read k_new, v_new; write K, V; min, max RMW

    # ---- outside the timed region: selection quality against Exact-TopK (replica 0, the first
    # decode steps), RocketKV's split against QUEST-like and SparQ-like settings of the same
    # approximation ratio (page_size * D / r)
    from sparse_kv_cache_snapkv_amd import quality
    ratio = w.page_size * D // w.r
    settings = dict(hybrid=(w.page_size, w.r), quest_like=(ratio, D), sparq_like=(1, max(1, D // ratio)))
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
    growing = dict(capacity=cap, appends=nsteps, append_us=round(grow_us["append"], 3),
                   append_bytes=app_bytes, append_plus_step_us=round(grow_us["append+step"], 3),
                   step_topk=tk_g, sync_status=rkv.decode_workspace_status(ws_g))

    # ---- outside the timed region: one layer of the 70B-shaped workload's eviction
    evict_70b = evict_70b_layer(rkv, torch)

    per_topk = {}
    stages_out = {}
    split_us = {name: ms * 1e3 / nsteps for name, ms in stage_ms.items() if name.startswith("split_")}
    for name, ms in stage_ms.items():
        kind, _, tk = name.partition("@")
        ab = algorithmic_bytes(w, int(tk) if tk else w.topk[0])
        if kind.startswith("split_"):
            continue
        if kind == "decode":
            us = ms * 1e3 / nsteps
            per_topk[tk] = dict(us_per_step=round(us, 3), algorithmic_bytes=ab["step"],
                                GBps=round(ab["step"] / (us * 1e-6) / 1e9, 1),
                                hbm_frac=round(ab["step"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4))
        else:
            nb = ab[kind] * R
            stages_out[name] = dict(us_total=round(ms * 1e3, 2), us_per_layer=round(ms * 1e3 / R, 2),
                                    algorithmic_bytes=nb, GBps=round(nb / (ms * 1e-3) / 1e9, 1))

    for tk in w.topk:
        ab = algorithmic_bytes(w, tk)
        a_us, t_us = split_us["split_approx"], split_us[f"split_topk@{tk}"]
        s_us = split_us[f"split_attend@{tk}"]
        per_topk[str(tk)]["three_calls"] = dict(
            approx_us=round(a_us, 3), approx_bytes=ab["approx"], topk_us=round(t_us, 3),
            topk_bytes=ab["topk"], attend_us=round(s_us, 3), attend_bytes=ab["attend"],
            sum_us=round(a_us + t_us + s_us, 3))

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
    stages = stages_out

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
        per_topk=per_topk, stages=stages, evict_70b_layer=evict_70b, growing_cache=growing,
        selection_quality=sel_q,
        roofline=roofline,
        sync_status=status,
        wall_ms_timed=round(wall_ms, 1))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_steps)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
