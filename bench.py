#!/usr/bin/env python3
"""Throughput of the prompt-token importance hot path on one MI355X.

A step is one pass of the whole path over one layer of seeded synthetic input
at the Mistral-7B / Llama-3.1-8B GQA shape (H_q = 32, H_kv = 8, d_k = 128,
W = 32 window queries) and L = 131072 prompt tokens:

  kvs_score (masked window softmax, column sums over rows and the 4 query
  heads of each KV head) -> kvs_select (page max + argmax, P = 16; cluster
  priority, theta = 2e-3, r = 3; top 1024 tokens per KV head with the
  cluster priority, window of 32 appended).

Inputs are resident in HBM before timing starts.  Four copies of K are rotated
so that no step finds its keys in the 256 MB Infinity Cache left warm by the
previous step.  The metric is prompt tokens scored per second (L per step).
The roofline object covers the longest kernel of the step, timed with HIP
events on the stream it runs on, between the parts of K further steps; its
algorithmic bytes are the bytes the method must move: K once, Q once, the
scores once.  The CPU baseline is the
fp64 oracle timed on the host on the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

NL = chr(10)
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=4, help="distinct K buffers cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--workload", default="mistral128k", choices=sorted(WORKLOADS),
                    help="mistral128k: the softmax window-score path at 128K (default); llama32k: the "
                         "same path at 32K with max-pool 7; cross32x16k: 32-layer cross-layer "
                         "aggregation at 16K; gemfilter128k and specprefill128k: the raw-logit paths; "
                         "delta32x8k: DELTA decode page sets; gather128k: compaction of the kept K and "
                         "V; chunksel128k: chunked-prefill block selection with cached key-block "
                         "means; chunksel128k_uncached: the same chunk recomputing every key-block mean")
    return ap.parse_args()


WORKLOADS = {
    # workload: (kernel-stats summary, traffic summary, kernel name fragment, kernel label)
    "mistral128k": ("kvs_mistral128k_kernel_stats.md", "score_fused_mistral128k_traffic.txt",
                    "score_fused", "score_fused_kernel (kvs_score, both passes in one launch)"),
    "llama32k": ("kvs_llama32k_kernel_stats.md", "score_fused_llama32k_traffic.txt",
                 "score_fused", "score_fused_kernel (kvs_score, both passes in one launch)"),
    "cross32x16k": ("kvs_cross32x16k_kernel_stats.md", "score_fused_cross32x16k_traffic.txt",
                    "score_fused", "32 x kvs_score (GROUP_SUM) + kvs_aggregate_layers (SUM_L1)"),
    "gemfilter128k": ("kvs_gemfilter128k_kernel_stats.md", "score_raw_gemfilter128k_traffic.txt",
                      "score_raw", "score_raw_kernel (kvs_score_raw, SUM over heads, W = 1)"),
    "specprefill128k": ("kvs_specprefill128k_kernel_stats.md", "score_raw_specprefill128k_traffic.txt",
                        "score_raw", "score_raw_kernel (kvs_score_raw, MAX over heads, W = 8)"),
    "delta32x8k": ("kvs_delta32x8k_kernel_stats.md", "delta_pages_delta32x8k_traffic.txt",
                   "delta", "kvs_delta_pages (delta_fused_kernel: logits, page scores and page sets in "
                            "one launch)"),
    "gather128k": ("kvs_gather128k_kernel_stats.md", "gather_gather128k_traffic.txt",
                   "gather_kernel", "gather_kernel (kvs_gather_kv, K and V)"),
    "chunksel128k": ("kvs_chunksel128k_kernel_stats.md", "block_topp_chunksel128k_traffic.txt",
                     "block_topp_kernel", "block_topp_kernel (kvs_block_select_cached)"),
    "chunksel128k_uncached": ("kvs_chunksel128k_uncached_kernel_stats.md",
                              "block_mean_chunksel128k_uncached_traffic.txt", "block_mean_kernel",
                              "kvs_block_select (every key-block mean from K: block_mean_kernel, "
                              "block_logits_kernel, block_topp_kernel)"),
}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", WORKLOADS["mistral128k"][1])


# Sources of each workload's roofline kernel(s), besides the shared header.
KERNEL_SOURCES = {
    "mistral128k": ("grid_sync.h", "score.hip"),
    "llama32k": ("grid_sync.h", "score.hip"),
    "cross32x16k": ("grid_sync.h", "score.hip"),
    "gemfilter128k": ("score.hip",),
    "specprefill128k": ("score.hip",),
    "delta32x8k": ("grid_sync.h", "score.hip", "select_ops.h", "topk.hip", "wave_ops.h"),
    "gather128k": ("gather.hip",),
    "chunksel128k": ("blocks.hip", "wave_ops.h"),
    "chunksel128k_uncached": ("blocks.hip", "wave_ops.h"),
}


def source_hash(workload=None):
    """sha256[:16] over HIP sources of the library, in name order: with a
    workload, the files of its roofline kernel plus the internal header (a
    counter summary taken on other sources of that kernel does not describe
    it); without one, every HIP source."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "prompt_token_importance_amd", "csrc")
    if workload is None:
        files = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    else:
        files = [os.path.join(csrc, f) for f in sorted(KERNEL_SOURCES[workload] + ("kvs_internal.h",))]
    h = hashlib.sha256()
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_summary(path=TRAFFIC_SUMMARY, workload="mistral128k"):
    """The key: value lines of a committed counter summary, or None when the
    summary is missing or was taken on another source of its kernel."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash(workload):
        return None
    return kv


def measured_traffic(path=TRAFFIC_SUMMARY, workload="mistral128k"):
    """HBM bytes per launch of the roofline kernel, or None (see traffic_summary)."""
    kv = traffic_summary(path, workload)
    try:
        return float(kv["traffic_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def cpu_baseline(ly, theta, r, budget, n_forced, P, min_seconds=10.0, max_reps=8):
    """The fp64 oracle, as it stands, on the full workload, one BLAS thread."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    n = ly.L - ly.W
    reps, t_total = 0, 0.0
    with threadpool_limits(limits=1):
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t0 = time.perf_counter()
            S = oracle.score(ly.Q, ly.K, L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv,
                             q_pos0=ly.q_pos0)
            z, arg = oracle.pages(S[:, :n], P, oracle.RED_MAX)
            prio = oracle.cluster_priority(z, arg, n, float(np.float32(theta)), r)
            oracle.topk(S[:, :n], budget, prio, n_forced)
            t_total += time.perf_counter() - t0
            reps += 1
    sec = t_total / reps
    return {"value": ly.L / sec, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"full workload (all 8 KV heads, L={ly.L}), {reps} repetition(s), "
                      f"{sec:.2f} s each; score + page max + cluster priority + top-k in float64 NumPy"}


def profile_commands(workload="mistral128k", out="profile_out"):
    """The rocprofv3 runs a workload's summaries come from, writing under `out`."""
    wl = "" if workload == "mistral128k" else f" --workload {workload}"
    d = "" if workload == "mistral128k" else f"_{workload}"
    base = "python3 bench.py --no-cpu-baseline --copy-calibration" + wl
    return {
        "trace": f"rocprofv3 --kernel-trace --stats -f csv -d {out}/trace{d} -o bench -- {base}",
        "FETCH_SIZE": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/pmc_FETCH_SIZE{d} -o bench -- "
                      f"{base} --steps 10 --warmup 2",
        "WRITE_SIZE": f"rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/pmc_WRITE_SIZE{d} -o bench -- "
                      f"{base} --steps 10 --warmup 2",
    }


WORKLOAD_TITLES = {
    "mistral128k": "Mistral-7B GQA layer at L = 131072, softmax window scores + cluster top-k",
    "llama32k": "Llama-3.1-8B GQA layer at L = 32768, softmax window scores + max-pool 7 top-k",
    "cross32x16k": "32 layers of the Llama-3.1-8B GQA shape at L = 16384, per-layer scores summed over "
                   "the heads, L1-normalised sum over layers, top 20%",
    "gemfilter128k": "Mistral-7B GQA layer at L = 131072, GemFilter raw last-token scores + pooled top-k",
    "specprefill128k": "Mistral-7B GQA layer at L = 131072, Speculative-Prefill raw scores (8 lookahead "
                       "queries) + mean, pool and top-k",
    "delta32x8k": "Llama-3.1-8B GQA Delta-layer decode step, 32 sequences x 8192 cached tokens, DELTA "
                  "page sets (P = 16, K = 64, L = 8)",
    "gather128k": "Mistral-7B GQA layer at L = 131072, K and V of the kept 20% of every KV head "
                  "gathered into compact arrays",
    "chunksel128k": "chunked prefill at L = 131072, last 1024-token chunk: cached key-block means, "
                    "block top-p 0.9 and the per-group page table",
    "chunksel128k_uncached": "chunked prefill at L = 131072, last 1024-token chunk: every key-block "
                             "mean from K, block top-p 0.9 and the per-group page table",
}


def summarize_profiles(out_dir, workload="mistral128k"):
    """Writes the committed profile summaries of one bench workload from rocprofv3 CSV output.

    profiles/kvs_<workload>_kernel_stats.md: per-kernel average durations;
    profiles/<kernel>_<workload>_traffic.txt: HBM bytes per launch of the
    roofline kernel from FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for the plain 256 MiB copy in the same run.
    """
    import csv
    import statistics as st

    stats_name, traffic_name, frag, label = WORKLOADS[workload]
    cmds = profile_commands(workload, os.path.normpath(out_dir))
    d = "" if workload == "mistral128k" else f"_{workload}"

    def short(name):
        for pre in ("void ", "kvs::(anonymous namespace)::"):
            name = name.replace(pre, "")
        return name.split("(")[0]

    stats = list(csv.DictReader(open(os.path.join(out_dir, f"trace{d}", "bench_kernel_stats.csv"))))
    lines = [f"# Kernel durations, {WORKLOAD_TITLES[workload]} (bench.py workload)", "",
             "Command (from the repository root, with rocprofv3 started in /tmp):", "",
             "    " + cmds["trace"], "",
             "Calls cover the warm-up steps, the timed steps and the event-timed steps.", "",
             "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    srcs = ", ".join(sorted(KERNEL_SOURCES[workload] + ("kvs_internal.h",)))
    lines += ["", f"Sources of the roofline kernel ({srcs}) sha256[:16]: {source_hash(workload)}", ""]
    open(os.path.join(ROOT, "profiles", stats_name), "w").write(NL.join(lines))

    def counter(name):
        rows = list(csv.DictReader(open(os.path.join(out_dir, f"pmc_{name}{d}", "bench_counter_collection.csv"))))
        per = {}
        for r in rows:
            n = r["Kernel_Name"]
            key = "kernel" if frag in n else "copy" if "copyBuffer" in n else None
            if key:
                per.setdefault(key, []).append(float(r["Counter_Value"]))
        out = {k: st.median(v) for k, v in per.items()}
        if workload == "chunksel128k_uncached":
            # the roofline covers the whole uncached select: the medians of the key-block
            # mean launch (over K), the query-block mean launch, the logits and the top-p
            means, parts = [], {}
            for r in rows:
                n = r["Kernel_Name"]
                if "block_mean_kernel" in n:
                    means.append(float(r["Counter_Value"]))
                for kn in ("block_logits_kernel", "block_topp_kernel"):
                    if kn in n:
                        parts.setdefault(kn, []).append(float(r["Counter_Value"]))
            cut = (min(means) + max(means)) / 2
            big = [v for v in means if v >= cut]
            small = [v for v in means if v < cut] or [0.0]
            out["kernel"] = (st.median(big) + st.median(small) +
                             sum(st.median(v) for v in parts.values()))
        if workload == "delta32x8k":
            # the roofline covers the whole call: the sum of its kernels' medians (one launch,
            # or the logits, page and selection kernels where that form does not apply)
            parts = {}
            for r in rows:
                n = r["Kernel_Name"]
                for kn in ("delta_fused_kernel", "delta_logits_kernel", "delta_page_kernel",
                           "topk_delta_kernel"):
                    if kn in n:
                        parts.setdefault(kn, []).append(float(r["Counter_Value"]))
            out["kernel"] = sum(st.median(v) for v in parts.values())
        return out

    fetch, write = counter("FETCH_SIZE"), counter("WRITE_SIZE")
    copy_kib = (256 << 20) / 1024
    f_fetch, f_write = copy_kib / fetch["copy"], copy_kib / write["copy"]
    traffic = (fetch["kernel"] * f_fetch + write["kernel"] * f_write) * 1024
    txt = [
        f"# HBM traffic of {label}, {WORKLOAD_TITLES[workload]}",
        "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, medians), each scaled by the same counter's",
        "# reading for a plain 256 MiB device copy (torch copy_) in the same run.",
        "# Commands (from the repository root, with rocprofv3 started in /tmp):",
        "#   " + cmds["FETCH_SIZE"],
        "#   " + cmds["WRITE_SIZE"],
        f"# source_sha256_16 covers {', '.join(sorted(KERNEL_SOURCES[workload] + ('kvs_internal.h',)))}",
        f"source_sha256_16: {source_hash(workload)}",
        f"copy_fetch_kib: {fetch['copy']:.1f}",
        f"copy_write_kib: {write['copy']:.1f}",
        f"fetch_scale: {f_fetch:.4f}",
        f"write_scale: {f_write:.4f}",
        f"kernel_fetch_kib: {fetch['kernel']:.1f}",
        f"kernel_write_kib: {write['kernel']:.1f}",
    ]
    txt += [f"traffic_bytes_per_launch: {traffic:.0f}", ""]
    open(os.path.join(ROOT, "profiles", traffic_name), "w").write(NL.join(txt))
    print(NL.join(lines[-6:]))
    print(NL.join(txt))


def copy_calibration(timed):
    import torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    copy_ms = timed(lambda j: dst.copy_(src))
    gbs = 2 * src.numel() / (copy_ms * 1e-3) / 1e9
    log(f"plain 256 MiB copy: {copy_ms * 1e3:.1f} us, {gbs:.0f} GB/s read+write")
    return gbs


def bench_raw(args):
    """Raw-logit workloads: one layer scored with kvs_score_raw, then the selection.

    gemfilter128k: the last prompt token's raw logits summed over all 32 heads
    -> kvs_select with average pooling k = 7 -> top 20% of the prompt.
    specprefill128k: 8 lookahead queries, max over all heads, combined into the
    running max over layers -> kvs_pool_pages (mean over the queries, average
    pooling k = 7) -> kvs_topk of 20%.  The step scores one layer and finalises,
    which a multi-layer caller would do once per prompt (a conservative step).
    """
    import ctypes
    import torch
    import synth
    import prompt_token_importance_amd as kvs

    lib = kvs.library()
    gem = args.workload == "gemfilter128k"
    t0 = time.perf_counter()
    ly = synth.last_token_layer() if gem else synth.lookahead_layer(0)
    L, W, d_k, H_q, H_kv = ly.L, ly.W, ly.d_k, ly.H_q, ly.H_kv
    budget = L // 5
    Q = kvs.bf16_from_bits(ly.Q)
    K0 = kvs.bf16_from_bits(ly.K)
    Ks = [K0] + [K0.clone() for _ in range(max(0, args.rotate - 1))]
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")
    reduce = kvs.RED_SUM if gem else kvs.RED_MAX
    acc = kvs.ACC_WRITE if gem else kvs.ACC_MAX
    ra = kvs.raw_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, reduce=reduce,
                      accumulate=acc)
    S = torch.zeros(W, L, dtype=torch.float32, device="cuda")
    pooled = torch.empty(1, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(1, budget, dtype=torch.int32, device="cuda")
    sel = kvs.select_args(budget=budget, pool=kvs.RED_MEAN, pool_k=7)
    ws_bytes = lib.kvs_select_workspace(1, L, budget) if gem else lib.kvs_topk_workspace(1, L, budget)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p
    pQ, pS, pP, pI, pW = V(Q.data_ptr()), V(S.data_ptr()), V(pooled.data_ptr()), V(idx.data_ptr()), V(ws.data_ptr())
    pKs = [V(k.data_ptr()) for k in Ks]
    rra, rsel = ctypes.byref(ra), ctypes.byref(sel)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = lib.kvs_score_raw(rra, pQ, pKs[i % len(pKs)], pS, sp)
        if ev is not None:
            ev[1].record(stream)
        if gem:
            st |= lib.kvs_select(pS, 1, L, L, rsel, pI, pW, ws_bytes, sp)
        else:
            st |= lib.kvs_pool_pages(pS, W, L, L, kvs.RED_MEAN, kvs.RED_MEAN, 7, 0, kvs.RED_SUM, pP,
                                     None, None, sp)
            st |= lib.kvs_topk(pP, 1, L, L, budget, None, 0, pI, None, pW, ws_bytes, sp)
        if ev is not None:
            ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"libkvs call failed in step {i}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    raw_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    sel_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    log(f"per step: {ms_step * 1e3:.1f} us wall; events: raw scores {raw_ms * 1e3:.1f} us, "
        f"selection {sel_ms * 1e3:.1f} us")

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(args.steps):
            fn(j)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    copy_gbs = copy_calibration(timed) if args.copy_calibration else None
    # Algorithmic bytes of one raw launch: K once, Q once, S written once (and
    # read once when combined with the running max over layers).
    alg_bytes = H_kv * L * d_k * 2 + H_q * W * d_k * 2 + W * L * 4 * (1 if acc == kvs.ACC_WRITE else 2)
    achieved = alg_bytes / (raw_ms * 1e-3) / 1e9
    stats_name, traffic_name, frag, label = WORKLOADS[args.workload]
    desc = ("gemfilter_last_token_128k: H_q=32 H_kv=8 d_k=128 L=131072 W=1; raw logits summed over "
            "heads -> average pool 7 -> top 20%" if gem else
            "specprefill_lookahead_128k: H_q=32 H_kv=8 d_k=128 L=131072 W=8 lookahead queries; raw "
            "logits max over heads into the running layer max -> mean over queries -> average pool 7 "
            "-> top 20%")
    out = {
        "metric": "prompt tokens scored/sec at L=128K, 8B GQA shape; % of HBM roofline",
        "value": L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "L": L, "W": W, "d_k": d_k, "H_q": H_q, "H_kv": H_kv,
                   "budget": budget, "k_buffers_rotated": len(Ks)},
        "roofline": {
            "kernel": label,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(os.path.join(ROOT, "profiles", traffic_name), args.workload),
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us": raw_ms * 1e3,
            "kernel_source_sha256_16": source_hash(args.workload),
            "event_us": {"raw_scores": raw_ms * 1e3, "selection": sel_ms * 1e3},
            "copy_256MiB_GBs": copy_gbs,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline_raw(ly, gem, budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_delta(args):
    """DELTA decode step at a Delta-layer for a batch: 32 sequences of 8192 cached
    tokens (Llama-3.1-8B heads), one decode query each -> kvs_delta_pages
    (per-head softmax, max over heads, page sums over P = 16, 8 recent pages +
    the top 56 older pages)."""
    import ctypes
    import torch
    import synth
    import prompt_token_importance_amd as kvs

    lib = kvs.library()
    B, L, H_q, H_kv, d_k, P, K_pages, L_recent = 32, 8192, 32, 8, 128, 16, 64, 8
    t0 = time.perf_counter()
    layers = [synth.gaussian_layer(700 + b, L=L, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L - 1,
                                   n_spans=8, span_len=64, lift=2.0, span_region=L - 1)
              for b in range(B)]
    import numpy as np
    Q = kvs.bf16_from_bits(np.stack([ly.Q[:, 0, :] for ly in layers]))
    Ks = [kvs.bf16_from_bits(ly.K) for ly in layers]
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s (K of the batch: "
        f"{sum(k.numel() for k in Ks) * 2 / 2**20:.0f} MiB, above the 256 MB cache)")
    ptrs = torch.tensor([k.data_ptr() for k in Ks], dtype=torch.int64, device="cuda")
    Lt = torch.full((B,), L, dtype=torch.int32, device="cuda")
    a = kvs.delta_args(B=B, d_k=d_k, H_q=H_q, H_kv=H_kv, L_max=L, P=P, K_pages=K_pages,
                       L_recent=L_recent)
    ws_bytes = kvs.kvs_delta_workspace(a)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    rho = torch.empty(B, K_pages, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p
    args_ = (ctypes.byref(a), V(Q.data_ptr()), V(ptrs.data_ptr()), V(Lt.data_ptr()), V(rho.data_ptr()),
             None, V(ws.data_ptr()), ws_bytes, sp)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        if lib.kvs_delta_pages(*args_) != 0:
            raise RuntimeError(f"kvs_delta_pages failed in step {i}")
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    log(f"per step: {ms_step * 1e3:.1f} us wall; events: kvs_delta_pages {call_ms * 1e3:.1f} us")

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(args.steps):
            fn(j)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    copy_gbs = copy_calibration(timed) if args.copy_calibration else None
    n_pages = (L + P - 1) // P
    # Algorithmic bytes of one call: every cached key once, the queries once,
    # the page sets written once.  The logits the implementation spills and
    # reads back (2 x 128 B per token) are not counted.
    alg_bytes = B * (H_kv * L * d_k * 2 + H_q * d_k * 2 + K_pages * 4)
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    stats_name, traffic_name, frag, label = WORKLOADS[args.workload]
    out = {
        "metric": "cached tokens scored/sec (DELTA decode page selection, batch 32 x 8K, 8B GQA shape); "
                  "% of HBM roofline",
        "value": B * L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "delta_decode_b32x8k: 32 sequences x 8192 cached tokens, H_q=32 H_kv=8 "
                               "d_k=128, one decode query each; per-head softmax -> max over heads -> "
                               "page sums P=16 -> 8 recent + top 56 pages",
                   "B": B, "L": L, "H_q": H_q, "H_kv": H_kv, "d_k": d_k, "P": P, "K_pages": K_pages,
                   "L_recent": L_recent, "n_pages": n_pages},
        "roofline": {
            "kernel": label,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(os.path.join(ROOT, "profiles", traffic_name), args.workload),
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us": call_ms * 1e3,
            "kernel_source_sha256_16": source_hash(args.workload),
            "copy_256MiB_GBs": copy_gbs,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline_delta(layers, L, d_k, H_q, H_kv, P, K_pages, L_recent)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def cpu_baseline_delta(layers, L, d_k, H_q, H_kv, P, K_pages, L_recent, min_seconds=10.0,
                       max_passes=8):
    """The fp64 oracle, as it stands, over the batch's sequences (repeated until
    min_seconds or max_passes passes), one BLAS thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    done, t_total = 0, 0.0
    with threadpool_limits(limits=1):
        while done < max_passes * len(layers) and (done < len(layers) or t_total < min_seconds):
            ly = layers[done % len(layers)]
            t0 = time.perf_counter()
            oracle.delta_pages(ly.Q[:, 0, :], ly.K, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, P=P,
                               K_pages=K_pages, L_recent=L_recent)
            t_total += time.perf_counter() - t0
            done += 1
    return {"value": done * L / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} sequence evaluations over the batch's {len(layers)} sequences "
                      f"({L} cached tokens each), {t_total / done * 1e3:.1f} ms each; softmax per "
                      "head, max, page sums, page top-k in float64 NumPy"}


def bench_gather(args):
    """KV compaction for a 128K-token Mistral-7B layer: every KV head keeps 20%
    of its tokens (ascending per-head lists, as kvs_select produces them), and
    K and V of the kept tokens are copied into [8][26214][128] arrays."""
    import ctypes
    import numpy as np
    import torch
    import synth
    import prompt_token_importance_amd as kvs

    lib = kvs.library()
    H, L, d = 8, 131072, 128
    n = L // 5
    t0 = time.perf_counter()
    ly = synth.mistral_layer()
    K = kvs.bf16_from_bits(ly.K)
    V = kvs.bf16_from_bits(np.ascontiguousarray(ly.K[:, ::-1, :]))   # another tensor of the same shape
    # per-head kept lists: the top 20% of seeded scores, ascending
    x = synth.score_array(77, H, L)
    idx = np.sort(np.argsort(-x, axis=1, kind="stable")[:, :n], axis=1).astype(np.int32)
    I = torch.from_numpy(idx).cuda()
    Ko = torch.empty(H, n, d, dtype=torch.bfloat16, device="cuda")
    Vo = torch.empty_like(Ko)
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V_ = ctypes.c_void_p
    call = (V_(K.data_ptr()), V_(V.data_ptr()), H, L, d, 0, 0, V_(I.data_ptr()), n, None, n, 1,
            V_(Ko.data_ptr()), V_(Vo.data_ptr()), sp)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        if lib.kvs_gather_kv(*call) != 0:
            raise RuntimeError(f"kvs_gather_kv failed in step {i}")
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    log(f"per step: {ms_step * 1e3:.1f} us wall; events: kvs_gather_kv {call_ms * 1e3:.1f} us")

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(args.steps):
            fn(j)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    copy_gbs = copy_calibration(timed) if args.copy_calibration else None
    # every kept row of K and V read once and written once, plus the lists
    alg_bytes = 2 * 2 * H * n * d * 2 + H * n * 4
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    stats_name, traffic_name, frag, label = WORKLOADS[args.workload]
    out = {
        "metric": "kept tokens gathered/sec (K and V, 20% of every KV head of a 128K layer); "
                  "% of HBM roofline",
        "value": H * n / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gather_keep20_128k: H_kv=8 L=131072 d_k=128, 26214 kept tokens per KV "
                               "head, K and V copied to [8][26214][128]", "H_kv": H, "L": L, "d_k": d,
                   "kept_per_head": n},
        "roofline": {
            "kernel": label,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(os.path.join(ROOT, "profiles", traffic_name), args.workload),
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us": call_ms * 1e3,
            "kernel_source_sha256_16": source_hash(args.workload),
            "copy_256MiB_GBs": copy_gbs,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline_gather(ly.K, idx, L, n)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def cpu_baseline_gather(Kbits, idx, L, n, min_seconds=10.0, max_reps=8):
    """The oracle's gather, as it stands, on the workload (K and V: twice per
    repetition), one thread."""
    import oracle
    reps, t_total = 0, 0.0
    while reps < max_reps and (reps == 0 or t_total < min_seconds):
        t0 = time.perf_counter()
        oracle.gather_kv(Kbits, L=L, indices=idx, n=n, idx_ld=n)
        oracle.gather_kv(Kbits, L=L, indices=idx, n=n, idx_ld=n)
        t_total += time.perf_counter() - t0
        reps += 1
    sec = t_total / reps
    return {"value": idx.shape[0] * n / sec, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"full workload (8 KV heads x {n} kept tokens, K and V), {reps} repetition(s), "
                      f"{sec:.2f} s each; NumPy row copies in Python loops"}


def bench_chunksel(args):
    """The last 1024-query chunk of a 131072-token chunked prefill (Llama-3.1-8B
    heads, blocks of 64): kvs_block_select_cached with the means of the 2032
    earlier key blocks cached, then kvs_block_union_pagetable.  The same chunk
    without the cache (kvs_block_select, every key block's mean recomputed from
    the 256 MiB of K) is timed beside it."""
    import ctypes
    import torch
    import synth
    import prompt_token_importance_amd as kvs

    lib = kvs.library()
    t0 = time.perf_counter()
    ch = synth.chunk_select()
    Qc = kvs.bf16_from_bits(ch.Qc)
    K = kvs.bf16_from_bits(ch.K)
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")
    blk = ch.block
    a = kvs.block_select_args(Lq=ch.Lq, L=ch.L, d_k=ch.d_k, H_q=ch.H_q, H_kv=ch.H_kv, q_pos0=ch.q_pos0,
                              block=blk)
    n_qb, n_kvb = ch.Lq // blk, ch.L // blk
    n_cached = ch.q_pos0 // blk
    Kb = torch.empty(ch.H_kv, n_kvb, ch.d_k, dtype=torch.float32, device="cuda")
    # the cache as the earlier chunks left it
    a_prev = kvs.block_select_args(Lq=blk, L=ch.q_pos0, d_k=ch.d_k, H_q=ch.H_q, H_kv=ch.H_kv,
                                   q_pos0=ch.q_pos0 - blk, block=blk, k_head_stride=ch.L * ch.d_k)
    kvs.kvs_block_select_cached(Qc[:, :blk].contiguous(), K, a_prev, Kb, 0)
    M = torch.empty(ch.H_q, n_qb, n_kvb, dtype=torch.uint8, device="cuda")
    ws_b = kvs.kvs_block_select_workspace(a)
    ws = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    G = ch.H_q // ch.H_kv
    indptr = torch.empty(ch.H_kv + 1, dtype=torch.int32, device="cuda")
    indices = torch.empty(ch.H_kv * n_kvb, dtype=torch.int32, device="cuda")
    uws_b = int(lib.kvs_block_union_workspace(ch.H_q, ch.H_kv, 0, n_kvb))
    uws = torch.empty(max(uws_b, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V_ = ctypes.c_void_p
    ra = ctypes.byref(a)
    pQ, pK, pKb, pM, pws = V_(Qc.data_ptr()), V_(K.data_ptr()), V_(Kb.data_ptr()), V_(M.data_ptr()), V_(ws.data_ptr())

    def select_cached():
        return lib.kvs_block_select_cached(ra, pQ, pK, pKb, n_kvb, n_cached, pM, pws, ws_b, sp)

    def select_full():
        return lib.kvs_block_select(ra, pQ, pK, pM, pws, ws_b, sp)

    def union():
        return lib.kvs_block_union_pagetable(pM, ch.H_q, ch.H_kv, 0, n_qb, n_kvb, V_(indptr.data_ptr()),
                                             V_(indices.data_ptr()), V_(uws.data_ptr()), uws_b, sp)

    def step(i, ev=None, full=False):
        if ev is not None:
            ev[0].record(stream)
        st = select_full() if full else select_cached()
        if ev is not None:
            ev[1].record(stream)
        st |= union()
        if ev is not None:
            ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"chunk selection failed in step {i}")

    uncached = args.workload == "chunksel128k_uncached"
    for i in range(args.warmup):
        step(i, full=uncached)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, full=uncached)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    sel_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    uni_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    for i in range(args.steps):
        step(i, evs[i], full=True)
    torch.cuda.synchronize()
    full_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    log(f"per step: {ms_step * 1e3:.1f} us wall; events: cached select {sel_ms * 1e3:.1f} us, "
        f"union {uni_ms * 1e3:.1f} us; uncached select {full_ms * 1e3:.1f} us")

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(args.steps):
            fn(j)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    if args.copy_calibration:
        copy_calibration(timed)
    # block_topp_kernel bound: per (head, query block) the n_kvb fp32 key-block
    # means (d_k floats each) are read and dotted with the query block mean
    flops = 2.0 * ch.H_q * n_qb * n_kvb * ch.d_k
    achieved = flops / (sel_ms * 1e-3) / 1e12
    stats_name, traffic_name, frag, label = WORKLOADS[args.workload]
    event_us = {"select_cached": sel_ms * 1e3, "union": uni_ms * 1e3,
                "select_uncached": full_ms * 1e3}
    if not uncached:
        roof = {
            "kernel": "kvs_block_select_cached (block means of the chunk and its new key blocks, "
                      "block_logits_kernel on fp32 MFMA, block_topp_kernel)",
            "bound": "mfma", "achieved": achieved, "peak": 157.3, "unit": "TFLOP/s",
            "frac": achieved / 157.3, "traffic": None, "kernel_us": sel_ms * 1e3,
        }
    else:
        # the uncached select is bound by reading K once for the key-block means:
        # K once, the chunk's queries once, the mask written once
        alg = ch.H_kv * ch.L * ch.d_k * 2 + ch.H_q * ch.Lq * ch.d_k * 2 + ch.H_q * n_qb * n_kvb
        gbs = alg / (full_ms * 1e-3) / 1e9
        roof = {
            "kernel": label, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic(os.path.join(ROOT, "profiles", traffic_name), args.workload),
            "alg_bytes_per_launch": alg, "kernel_us": full_ms * 1e3,
        }
    roof.update({"kernel_source_sha256_16": source_hash(args.workload), "event_us": event_us})
    out = {
        "metric": "KV tokens covered/sec (chunked-prefill block selection, last chunk at L=128K); "
                  + ("% of fp32 matrix roofline" if not uncached else "% of HBM roofline"),
        "value": ch.L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if not uncached else "bf16",
        "data": "synthetic",
        "config": {"workload": "chunk_select_128k_last_chunk: K [8][131072][128], chunk Q [32][1024][128], "
                               "block 64, top-p 0.9, " + ("cached means of 2032 earlier blocks"
                                                          if not uncached else
                                                          "every key-block mean recomputed from K")
                               + " -> union page table", "L": ch.L, "Lq": ch.Lq, "block": blk,
                   "n_cached_blocks": 0 if uncached else n_cached},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline_chunksel(ch)
    print(json.dumps(out), flush=True)


def cpu_baseline_chunksel(ch, min_seconds=10.0, max_reps=8):
    """The oracle's block selection and union on the same chunk, one BLAS thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    reps, t_total = 0, 0.0
    with threadpool_limits(limits=1):
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t0 = time.perf_counter()
            M = oracle.block_select(ch.Qc, ch.K, Lq=ch.Lq, L=ch.L, d_k=ch.d_k, H_q=ch.H_q,
                                       H_kv=ch.H_kv, q_pos0=ch.q_pos0, block=ch.block)
            oracle.block_union_pagetable(M, H_q=ch.H_q, H_kv=ch.H_kv)
            t_total += time.perf_counter() - t0
            reps += 1
    sec = t_total / reps
    return {"value": ch.L / sec, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"full workload (the chunk, all heads), {reps} repetition(s), {sec:.2f} s each; "
                      "block means, top-p and union in float64 NumPy"}


def cpu_baseline_raw(ly, gem, budget, min_seconds=10.0, max_reps=8):
    """The fp64 oracle, as it stands, on the full raw-logit workload, one BLAS thread."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    L = ly.L
    reps, t_total = 0, 0.0
    with threadpool_limits(limits=1):
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t0 = time.perf_counter()
            R = oracle.score_raw(ly.Q, ly.K, L=L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv,
                                 reduce=oracle.RED_SUM if gem else oracle.RED_MAX)
            y = oracle.pool(R, oracle.RED_MEAN, 7) if gem else oracle.aggregate_raw([R], pool_k=7)[None, :]
            oracle.topk(y, budget)
            t_total += time.perf_counter() - t0
            reps += 1
    sec = t_total / reps
    return {"value": L / sec, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"full workload (one layer, all 32 heads, L={L}), {reps} repetition(s), "
                      f"{sec:.2f} s each; raw scores + pooling + top-k in float64 NumPy"}


def cpu_info():
    """CPU model and the cores this process may use (capped at the 16 a one-GPU machine shares)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_layer_scores(ly, heads, threads):
    """oracle.score on one layer, its KV groups spread over `threads` Python threads
    (NumPy releases the GIL in its kernels; each call uses one BLAS thread)."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    G = ly.H_q // ly.H_kv

    def one(g):
        return oracle.score(ly.Q[g * G:(g + 1) * G], ly.K[g:g + 1], L=ly.L, W=ly.W, d_k=ly.d_k,
                            H_q=G, H_kv=1, q_pos0=ly.q_pos0, heads=heads)

    if threads <= 1:
        parts = [one(g) for g in range(ly.H_kv)]
    else:
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(one, range(ly.H_kv)))
    return np.concatenate(parts, axis=0)


def cpu_baseline_softmax(ly, sel, min_seconds=5.0, max_reps=8):
    """The fp64 oracle as it stands on the full layer: scores (KV groups in parallel
    threads), then the selection rows; timed with all cores and with one."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    n = ly.L - ly.W

    def run(threads):
        S = oracle_layer_scores(ly, oracle.HEADS_GROUP_SUM, threads)[:, :n]
        if sel["kind"] == "cluster":
            z, arg = oracle.pages(S, sel["P"], oracle.RED_MAX)
            prio = oracle.cluster_priority(z, arg, n, float(np.float32(sel["theta"])), sel["r"])
            oracle.topk(S, sel["budget"], prio, ly.W)
        else:
            y = oracle.pool(S, oracle.RED_MAX, sel["pool_k"])
            oracle.topk(y, sel["budget"], None, ly.W)

    def timed(threads):
        reps, t_total = 0, 0.0
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t0 = time.perf_counter()
            run(threads)
            t_total += time.perf_counter() - t0
            reps += 1
        return t_total / reps, reps

    model, cores = cpu_info()
    used = min(cores, ly.H_kv)
    with threadpool_limits(limits=1):
        sec_all, reps_all = timed(used)
        sec_one, reps_one = timed(1)
    return {"value": ly.L / sec_all, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"full workload (all {ly.H_kv} KV heads, L={ly.L}); {reps_all} repetition(s) of "
                      f"{sec_all:.2f} s on {used} threads (one per KV group), {reps_one} of "
                      f"{sec_one:.2f} s on one; score + selection in float64 NumPy",
            "one_core_value": ly.L / sec_one, "cpu_model": model, "cores_available": cores}


def bench_softmax(args):
    """The softmax window-score path on one layer: kvs_score (both passes, one
    launch), then kvs_select.  mistral128k: page max P = 16 + cluster priority (theta =
    2e-3, r = 3) + top 1024 per KV head with the window; llama32k: max-pool 7 +
    top 1024 per KV head with the window."""
    import torch
    import synth
    import prompt_token_importance_amd as kvs

    lib = kvs.library()
    mistral = args.workload == "mistral128k"
    t0 = time.perf_counter()
    ly = synth.mistral_layer() if mistral else synth.llama_layer()
    L, W, d_k, H_q, H_kv = ly.L, ly.W, ly.d_k, ly.H_q, ly.H_kv
    n = L - W
    budget, n_forced = 1024, W
    # K buffers cycled so no step finds its keys warm in the 256 MB Infinity Cache
    rotate = args.rotate if mistral else max(args.rotate, 8)
    Q = kvs.bf16_from_bits(ly.Q)
    K0 = kvs.bf16_from_bits(ly.K)
    Ks = [K0] + [K0.clone() for _ in range(max(0, rotate - 1))]
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")

    a0 = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0)
    a1 = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, phase=1)
    a2 = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, phase=2)
    ws_bytes = kvs.kvs_score_workspace(a0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    S = torch.empty(H_kv, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(H_kv, budget + n_forced, dtype=torch.int32, device="cuda")
    if mistral:
        sel = {"kind": "cluster", "P": 16, "theta": 2e-3, "r": 3, "budget": budget}
        sel_args = kvs.select_args(budget=budget, n_forced=n_forced, cluster_P=16,
                                   cluster_theta=2e-3, cluster_r=3)
    else:
        sel = {"kind": "pool", "pool_k": 7, "budget": budget}
        sel_args = kvs.select_args(budget=budget, n_forced=n_forced, pool=kvs.RED_MAX, pool_k=7)
    tk_bytes = lib.kvs_select_workspace(H_kv, n, budget)
    tk_ws = torch.empty(max(tk_bytes, 1), dtype=torch.uint8, device="cuda")

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p
    pQ, pS, pws = V(Q.data_ptr()), V(S.data_ptr()), V(ws.data_ptr())
    pKs = [V(k.data_ptr()) for k in Ks]
    pidx = V(idx.data_ptr())
    ptk = V(tk_ws.data_ptr())
    ra0, ra1, ra2, rsel = (ctypes.byref(a0), ctypes.byref(a1), ctypes.byref(a2),
                           ctypes.byref(sel_args))

    def step(i, ev=None):
        pK = pKs[i % len(pKs)]
        if ev is not None:
            ev[0].record(stream)
        st = lib.kvs_score(ra0, pQ, pK, pS, pws, ws_bytes, sp)
        if ev is not None:
            ev[1].record(stream)
        st |= lib.kvs_select(pS, H_kv, n, L, rsel, pidx, ptk, tk_bytes, sp)
        if ev is not None:
            ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"libkvs call failed in step {i}")

    def two_launch(i, ev):
        """The score as its two phase calls (one launch per pass), for comparison."""
        pK = pKs[i % len(pKs)]
        ev[0].record(stream)
        st = lib.kvs_score(ra1, pQ, pK, pS, pws, ws_bytes, sp)
        ev[1].record(stream)
        st |= lib.kvs_score(ra2, pQ, pK, pS, pws, ws_bytes, sp)
        ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"libkvs call failed in step {i}")

    # Timed region: K whole steps, bracketed by synchronizations, no events
    # inside (an event record idles the GPU for a few microseconds).
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps
    # Kernel timing: K more steps with HIP events on the launch stream between
    # the parts of each step, so every kernel is timed under the same
    # conditions (clock, caches, neighbours) as in the timed region.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        two_launch(args.warmup + 2 * args.steps + i, ev2[i])
    torch.cuda.synchronize()

    def part(evl, a):
        return sum(ev[a].elapsed_time(ev[a + 1]) for ev in evl) / args.steps

    score, select = part(evs, 0), part(evs, 1)
    pass1, pass2 = part(ev2, 0), part(ev2, 1)
    step_us = sorted(ev[0].elapsed_time(ev[2]) * 1e3 for ev in evs)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(args.steps):
            fn(j)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    log(f"per step: {ms_step * 1e3:.1f} us wall; events: score {score * 1e3:.1f} us (one launch; "
        f"as two launches: pass1 {pass1 * 1e3:.1f} us, pass2 {pass2 * 1e3:.1f} us), "
        f"select {select * 1e3:.1f} us")
    copy_gbs = copy_calibration(timed) if args.copy_calibration else None

    # Algorithmic bytes of the layer (and of one score launch): K once, Q once,
    # S written once -> 2048 + 32 + ~2 bytes per token.  The two-pass design
    # streams K twice: its bytes, and the time at which they would move at 70%
    # of the HBM peak, are reported beside.
    k_bytes = H_kv * L * d_k * 2
    q_bytes = H_q * W * d_k * 2
    s_bytes = H_kv * L * 4
    alg_bytes = k_bytes + q_bytes + s_bytes
    two_pass_bytes = 2 * k_bytes + q_bytes + s_bytes
    dom_ms = score
    achieved = alg_bytes / (dom_ms * 1e-3) / 1e9
    stats_name, traffic_name, frag, label = WORKLOADS[args.workload]
    tpath = os.path.join(ROOT, "profiles", traffic_name)
    traffic = measured_traffic(tpath, args.workload)
    counter_gbs = traffic / (dom_ms * 1e-3) / 1e9 if traffic else None
    flops = 2 * 2.0 * H_q * W * L * d_k   # both passes multiply the window rows by K
    tag = "128K" if mistral else "32K"
    out = {
        "metric": f"prompt tokens scored/sec at L={tag}, 8B GQA shape; % of HBM roofline",
        "value": L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "event_step_us_p50_p90": [step_us[len(step_us) // 2],
                                  step_us[min(len(step_us) - 1, (9 * len(step_us)) // 10)]],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("mistral7b_gqa_layer_128k: H_q=32 H_kv=8 d_k=128 L=131072 W=32; score -> page "
                         "max P=16 -> cluster theta=2e-3 r=3 -> top-1024 + 32 window per KV head"
                         if mistral else
                         "llama31_8b_gqa_layer_32k: H_q=32 H_kv=8 d_k=128 L=32768 W=32; score -> max-pool 7 "
                         "-> top-1024 + 32 window per KV head"),
            "L": L, "W": W, "d_k": d_k, "H_q": H_q, "H_kv": H_kv, "budget": budget,
            "k_buffers_rotated": len(Ks),
        },
        "roofline": {
            "kernel": label,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us": dom_ms * 1e3,
            "mfma_frac": flops / (dom_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "kernel_source_sha256_16": source_hash(args.workload),
            "event_us": {"score_one_launch": score * 1e3, "selection": select * 1e3,
                         "two_launch_pass1_stats": pass1 * 1e3,
                         "two_launch_pass2_colsum": pass2 * 1e3},
            "copy_256MiB_GBs": copy_gbs,
            # the layer's algorithmic bytes (K once) over the score launch (both passes; the
            # same figure as frac) and over the whole step
            "alg_frac_score_pair": alg_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_frac_step": alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            # the score launch's bytes from the counter runs over its time
            "score_passes_counter_GBs": counter_gbs,
            "score_passes_counter_frac": counter_gbs / HBM_PEAK_GBS if counter_gbs else None,
            # K twice, Q and S once: the bytes of a two-pass design over the launch's time,
            # and the launch time at which they move at 70% of the peak
            "two_pass_bytes": two_pass_bytes,
            "two_pass_frac": two_pass_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "two_pass_us_at_70pct": two_pass_bytes / (0.7 * HBM_PEAK_GBS * 1e9) * 1e6,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline_softmax(ly, sel)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def bench_cross(args):
    """Cross-layer aggregation over 32 layers of the Llama-3.1-8B GQA shape at
    L = 16384: each layer's window scores per KV group (kvs_score GROUP_SUM,
    phase 0), summed over the groups, L1-normalised and added over the layers
    by kvs_aggregate_layers (SUM_L1, which sums its H rows first), then the top
    20% of the tokens (kvs_topk).  A step is the whole 32-layer pass; tokens/s =
    32 * L / t."""
    import torch
    import synth
    import prompt_token_importance_amd as kvs

    lib = kvs.library()
    n_layers, L = 32, 16384
    t0 = time.perf_counter()
    layers = [synth.cross_layer(l, L=L) for l in range(n_layers)]
    W, d_k, H_q, H_kv = layers[0].W, layers[0].d_k, layers[0].H_q, layers[0].H_kv
    Qs = [kvs.bf16_from_bits(ly.Q) for ly in layers]
    Ks = [kvs.bf16_from_bits(ly.K) for ly in layers]
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s (K of the 32 layers: "
        f"{sum(k.numel() for k in Ks) * 2 / 2**20:.0f} MiB)")
    budget = (2 * L) // 10
    a = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=layers[0].q_pos0,
                       heads=kvs.HEADS_GROUP_SUM)
    ws_bytes = kvs.kvs_score_workspace(a)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    row = torch.empty(H_kv, L, dtype=torch.float32, device="cuda")
    acc = torch.empty(1, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(1, budget, dtype=torch.int32, device="cuda")
    ag_bytes = lib.kvs_aggregate_workspace(L)
    ag_ws = torch.empty(max(ag_bytes, 1), dtype=torch.uint8, device="cuda")
    tk_bytes = lib.kvs_topk_workspace(1, L, budget)
    tk_ws = torch.empty(max(tk_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p
    ra = ctypes.byref(a)
    pQs = [V(q.data_ptr()) for q in Qs]
    pKs = [V(k.data_ptr()) for k in Ks]
    prow, pacc, pws, pag, ptk, pidx = (V(row.data_ptr()), V(acc.data_ptr()), V(ws.data_ptr()),
                                       V(ag_ws.data_ptr()), V(tk_ws.data_ptr()), V(idx.data_ptr()))

    def step(i, ev=None):
        st = 0
        if ev is not None:
            ev[0].record(stream)
        for l in range(n_layers):
            st |= lib.kvs_score(ra, pQs[l], pKs[l], prow, pws, ws_bytes, sp)
            st |= lib.kvs_aggregate_layers(pacc, prow, H_kv, L, L, kvs.RED_SUM_L1, int(l == 0), pag,
                                           ag_bytes, sp)
        if ev is not None:
            ev[1].record(stream)
        st |= lib.kvs_topk(pacc, 1, L, L, budget, None, 0, pidx, None, ptk, tk_bytes, sp)
        if ev is not None:
            ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"libkvs call failed in step {i}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    layers_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    topk_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    log(f"per step: {ms_step * 1e3:.1f} us wall; events: 32 layers (score + aggregate) "
        f"{layers_ms * 1e3:.1f} us, top-k {topk_ms * 1e3:.1f} us")

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(args.steps):
            fn(j)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    copy_gbs = copy_calibration(timed) if args.copy_calibration else None
    # algorithmic bytes of the 32-layer pass: every layer's K and Q once, one score row per
    # KV group and layer
    alg_bytes = n_layers * (H_kv * L * d_k * 2 + H_q * W * d_k * 2 + H_kv * L * 4)
    achieved = alg_bytes / (layers_ms * 1e-3) / 1e9
    stats_name, traffic_name, frag, label = WORKLOADS[args.workload]
    out = {
        "metric": "prompt tokens scored/sec, 32-layer cross-layer aggregation at L=16K, 8B GQA shape; "
                  "% of HBM roofline",
        "value": n_layers * L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "cross_layer_32x16k: 32 layers, H_q=32 H_kv=8 d_k=128 L=16384 W=32; "
                               "per-layer score per KV group, summed over the groups -> L1-normalised "
                               "sum over layers -> top 20% (3276)", "layers": n_layers, "L": L, "W": W,
                   "budget": budget},
        "roofline": {
            "kernel": label,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us": layers_ms * 1e3,
            "kernel_source_sha256_16": source_hash(args.workload),
            "event_us": {"layers_score_and_aggregate": layers_ms * 1e3, "topk": topk_ms * 1e3},
            "copy_256MiB_GBs": copy_gbs,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline_cross(layers, budget)
    print(json.dumps(out), flush=True)


def cpu_baseline_cross(layers, budget, min_seconds=0.0):
    """The oracle on the 32-layer pass: per-layer scores (KV groups in threads),
    L1-normalised sum, top-k; all cores and one."""
    import oracle
    from threadpoolctl import threadpool_limits
    L = layers[0].L

    def run(threads):
        per = [oracle_layer_scores(ly, oracle.HEADS_ALL_SUM, threads) for ly in layers]
        agg = oracle.aggregate_layers(per, oracle.RED_SUM_L1)
        oracle.topk(agg[None, :], budget)

    model, cores = cpu_info()
    used = min(cores, layers[0].H_kv)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        run(used)
        sec_all = time.perf_counter() - t0
        t0 = time.perf_counter()
        run(1)
        sec_one = time.perf_counter() - t0
    n = len(layers) * L
    return {"value": n / sec_all, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"full workload ({len(layers)} layers x {L} tokens), one pass of {sec_all:.2f} s "
                      f"on {used} threads and one of {sec_one:.2f} s on one; float64 NumPy",
            "one_core_value": n / sec_one, "cpu_model": model, "cores_available": cores}


def main():
    if len(sys.argv) in (3, 4) and sys.argv[1] == "--summarize-profiles":
        summarize_profiles(sys.argv[2], *sys.argv[3:])
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no collectives; it would shard by KV head, every GPU running the same "
              "kernels on its share of the heads).")
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)")
        sys.exit(1)
    if args.workload in ("mistral128k", "llama32k"):
        bench_softmax(args)
    elif args.workload == "cross32x16k":
        bench_cross(args)
    elif args.workload == "delta32x8k":
        bench_delta(args)
    elif args.workload == "gather128k":
        bench_gather(args)
    elif args.workload in ("chunksel128k", "chunksel128k_uncached"):
        bench_chunksel(args)
    else:
        bench_raw(args)


if __name__ == "__main__":
    main()
