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
    return ap.parse_args()


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "score_colsum_mistral128k_traffic.txt")
SCORE_SOURCE = os.path.join(ROOT, "prompt_token_importance_amd", "csrc", "score.hip")


def source_hash():
    import hashlib
    return hashlib.sha256(open(SCORE_SOURCE, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per column-sum launch from the committed counter summary, or
    None when the summary is missing or was taken on another kernel source."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    kv = {}
    for line in open(TRAFFIC_SUMMARY):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
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


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/trace -o bench -- "
             "python3 bench.py --no-cpu-baseline --copy-calibration",
    "FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_FETCH_SIZE -o bench -- "
                  "python3 bench.py --no-cpu-baseline --copy-calibration --steps 10 --warmup 2",
    "WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_WRITE_SIZE -o bench -- "
                  "python3 bench.py --no-cpu-baseline --copy-calibration --steps 10 --warmup 2",
}


def summarize_profiles(out_dir):
    """Writes the committed profile summaries from rocprofv3 CSV output.

    profiles/kvs_mistral128k_kernel_stats.md: per-kernel average durations;
    profiles/score_colsum_mistral128k_traffic.txt: HBM bytes per column-sum
    launch from FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
    reads for the plain 256 MiB copy in the same run.
    """
    import csv
    import statistics as st

    def short(name):
        for pre in ("void ", "kvs::(anonymous namespace)::"):
            name = name.replace(pre, "")
        return name.split("(")[0]

    stats = list(csv.DictReader(open(os.path.join(out_dir, "trace", "bench_kernel_stats.csv"))))
    lines = ["# Kernel durations, Mistral-7B GQA layer at L = 131072 (bench.py workload)", "",
             "Command (repo root on the GPU box, cd /tmp first):", "",
             "    " + PROFILE_COMMANDS["trace"], "",
             "Calls cover the warm-up steps, the timed steps and the event-timed steps.", "",
             "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    lines += ["", f"Kernel source sha256[:16] of score.hip: {source_hash()}", ""]
    open(os.path.join(ROOT, "profiles", "kvs_mistral128k_kernel_stats.md"), "w").write(NL.join(lines))

    def counter(name):
        rows = list(csv.DictReader(open(os.path.join(out_dir, f"pmc_{name}", "bench_counter_collection.csv"))))
        per = {}
        for r in rows:
            n = r["Kernel_Name"]
            key = ("colsum" if "score_colsum" in n else "stats" if "score_stats" in n else
                   "copy" if "copyBuffer" in n else None)
            if key:
                per.setdefault(key, []).append(float(r["Counter_Value"]))
        return {k: st.median(v) for k, v in per.items()}

    fetch, write = counter("FETCH_SIZE"), counter("WRITE_SIZE")
    copy_kib = (256 << 20) / 1024
    f_fetch, f_write = copy_kib / fetch["copy"], copy_kib / write["copy"]
    traffic = (fetch["colsum"] * f_fetch + write["colsum"] * f_write) * 1024
    txt = [
        "# HBM traffic of score_colsum_kernel (kvs_score column-sum pass), Mistral-7B GQA layer, L = 131072",
        "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, medians), each scaled by the same counter's",
        "# reading for a plain 256 MiB device copy (torch copy_) in the same run.",
        "# Commands (repo root on the GPU box, cd /tmp first):",
        "#   " + PROFILE_COMMANDS["FETCH_SIZE"],
        "#   " + PROFILE_COMMANDS["WRITE_SIZE"],
        f"source_sha256_16: {source_hash()}",
        f"copy_fetch_kib: {fetch['copy']:.1f}",
        f"copy_write_kib: {write['copy']:.1f}",
        f"fetch_scale: {f_fetch:.4f}",
        f"write_scale: {f_write:.4f}",
        f"colsum_fetch_kib: {fetch['colsum']:.1f}",
        f"colsum_write_kib: {write['colsum']:.1f}",
        f"stats_fetch_kib: {fetch['stats']:.1f}",
        f"stats_write_kib: {write['stats']:.1f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        "",
    ]
    open(TRAFFIC_SUMMARY, "w").write(NL.join(txt))
    print(NL.join(lines[-6:]))
    print(NL.join(txt))


def main():
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-profiles":
        summarize_profiles(sys.argv[2])
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no collectives; see DESIGN.md for how it would shard).")
        sys.exit(2)

    import torch
    import synth
    import prompt_token_importance_amd as kvs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)")
        sys.exit(1)
    lib = kvs.library()

    # ------------------------------------------------------------ workload
    t0 = time.perf_counter()
    ly = synth.mistral_layer()
    L, W, d_k, H_q, H_kv = ly.L, ly.W, ly.d_k, ly.H_q, ly.H_kv
    n = L - W
    P, theta, r, budget, n_forced = 16, 2e-3, 3, 1024, W
    Q = kvs.bf16_from_bits(ly.Q)
    K0 = kvs.bf16_from_bits(ly.K)
    Ks = [K0] + [K0.clone() for _ in range(max(0, args.rotate - 1))]
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")

    a1 = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, phase=1)
    a2 = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, phase=2)
    ws_bytes = kvs.kvs_score_workspace(a1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    S = torch.empty(H_kv, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(H_kv, budget + n_forced, dtype=torch.int32, device="cuda")
    sel_args = kvs.select_args(budget=budget, n_forced=n_forced, cluster_P=P, cluster_theta=theta,
                               cluster_r=r)
    tk_bytes = lib.kvs_select_workspace(H_kv, n, budget)
    tk_ws = torch.empty(max(tk_bytes, 1), dtype=torch.uint8, device="cuda")

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p
    pQ, pS, pws = V(Q.data_ptr()), V(S.data_ptr()), V(ws.data_ptr())
    pKs = [V(k.data_ptr()) for k in Ks]
    pidx = V(idx.data_ptr())
    ptk = V(tk_ws.data_ptr())
    ra1, ra2, rsel = ctypes.byref(a1), ctypes.byref(a2), ctypes.byref(sel_args)

    def step(i, ev=None):
        pK = pKs[i % len(pKs)]
        if ev is not None:
            ev[0].record(stream)
        st = lib.kvs_score(ra1, pQ, pK, pS, pws, ws_bytes, sp)
        if ev is not None:
            ev[1].record(stream)
        st |= lib.kvs_score(ra2, pQ, pK, pS, pws, ws_bytes, sp)
        if ev is not None:
            ev[2].record(stream)
        st |= lib.kvs_select(pS, H_kv, n, L, rsel, pidx, ptk, tk_bytes, sp)
        if ev is not None:
            ev[3].record(stream)
        if st != 0:
            raise RuntimeError(f"libkvs call failed in step {i}")

    # ------------------------------------------------------------ timing
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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()

    def part(a):
        return sum(ev[a].elapsed_time(ev[a + 1]) for ev in evs) / args.steps

    pass1, pass2, select = part(0), part(1), part(2)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(args.steps):
            fn(j)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    log(f"per step: {ms_step * 1e3:.1f} us wall; events: score pass1+merge {pass1 * 1e3:.1f} us, "
        f"pass2 {pass2 * 1e3:.1f} us, select {select * 1e3:.1f} us")
    copy_gbs = None
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(2):
            dst.copy_(src)
        copy_ms = timed(lambda j: dst.copy_(src))
        copy_gbs = 2 * src.numel() / (copy_ms * 1e-3) / 1e9
        log(f"plain 256 MiB copy: {copy_ms * 1e3:.1f} us, {copy_gbs:.0f} GB/s read+write")

    # Algorithmic bytes of one column-sum launch: K once, Q once, S written once,
    # per-row constants (negligible) -> 2048 + 32 + ~2 bytes per token.
    k_bytes = H_kv * L * d_k * 2
    q_bytes = H_q * W * d_k * 2
    s_bytes = H_kv * L * 4
    alg_bytes = k_bytes + q_bytes + s_bytes
    dom_ms = pass2
    achieved = alg_bytes / (dom_ms * 1e-3) / 1e9
    flops = 2.0 * H_q * W * L * d_k
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
        "config": {
            "workload": "mistral7b_gqa_layer_128k: H_q=32 H_kv=8 d_k=128 L=131072 W=32; "
                        "score -> page max P=16 -> cluster theta=2e-3 r=3 -> top-1024 + 32 window per KV head",
            "L": L, "W": W, "d_k": d_k, "H_q": H_q, "H_kv": H_kv, "budget": budget,
            "k_buffers_rotated": len(Ks),
        },
        "roofline": {
            "kernel": "score_colsum_kernel (kvs_score column-sum pass)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us": dom_ms * 1e3,
            "mfma_frac": flops / (dom_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "kernel_source_sha256_16": source_hash(),
            "event_us": {"score_pass1_stats_and_merge": pass1 * 1e3, "score_pass2_colsum": pass2 * 1e3,
                         "page_cluster_topk": select * 1e3},
            "copy_256MiB_GBs": copy_gbs,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(ly, theta, r, budget, n_forced, P)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
