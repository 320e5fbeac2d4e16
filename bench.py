#!/usr/bin/env python3
"""Throughput of the prompt-token importance hot path on one MI355X.

A step is one pass of the whole path over one layer of seeded synthetic input
at the Mistral-7B / Llama-3.1-8B GQA shape (H_q = 32, H_kv = 8, d_k = 128,
W = 32 window queries) and L = 131072 prompt tokens:

  kvs_score (masked window softmax, column sums over rows and the 4 query
  heads of each KV head) -> kvs_pool_pages (page max + argmax, P = 16) ->
  kvs_cluster_priority (theta = 2e-3, r = 3) -> kvs_topk (1024 tokens per KV
  head with cluster priority, window of 32 appended).

Inputs are resident in HBM before timing starts.  Four copies of K are rotated
so that no step finds its keys in the 256 MB Infinity Cache left warm by the
previous step.  The metric is prompt tokens scored per second (L per step).
The roofline object covers the longest kernel of the step, timed with HIP
events on the stream it runs on; its algorithmic bytes are the bytes the
method must move: K once, Q once, the scores once.  The CPU baseline is the
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
    return ap.parse_args()


def cpu_baseline(ly, theta, r, budget, n_forced, P, min_seconds=10.0, max_reps=3):
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


def main():
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
    n_pages = (n + P - 1) // P
    Q = kvs.bf16_from_bits(ly.Q)
    K0 = kvs.bf16_from_bits(ly.K)
    Ks = [K0] + [K0.clone() for _ in range(max(0, args.rotate - 1))]
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s")

    a1 = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, phase=1)
    a2 = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, phase=2)
    ws_bytes = kvs.kvs_score_workspace(a1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    S = torch.empty(H_kv, L, dtype=torch.float32, device="cuda")
    page = torch.empty(H_kv, n_pages, dtype=torch.float32, device="cuda")
    parg = torch.empty(H_kv, n_pages, dtype=torch.int32, device="cuda")
    prio = torch.empty(H_kv, n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(H_kv, budget + n_forced, dtype=torch.int32, device="cuda")
    tk_bytes = lib.kvs_topk_workspace(H_kv, n, budget)
    tk_ws = torch.empty(max(tk_bytes, 1), dtype=torch.uint8, device="cuda")

    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = ctypes.c_void_p
    pQ, pS, pws = V(Q.data_ptr()), V(S.data_ptr()), V(ws.data_ptr())
    pKs = [V(k.data_ptr()) for k in Ks]
    ppage, parg_p, pprio, pidx = V(page.data_ptr()), V(parg.data_ptr()), V(prio.data_ptr()), V(idx.data_ptr())
    ptk = V(tk_ws.data_ptr())
    ra1, ra2 = ctypes.byref(a1), ctypes.byref(a2)
    theta_f = ctypes.c_float(theta)

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
        st |= lib.kvs_pool_pages(pS, H_kv, n, L, kvs.RED_NONE, kvs.RED_NONE, 7, P, kvs.RED_MAX,
                                 None, ppage, parg_p, sp)
        st |= lib.kvs_cluster_priority(ppage, parg_p, H_kv, n_pages, P, n, theta_f, r, pprio, sp)
        st |= lib.kvs_topk(pS, H_kv, n, L, budget, pprio, n_forced, pidx, ptk, tk_bytes, sp)
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
    # Kernel timing: the same steps again with HIP events on the stream around
    # the statistics pass, the column-sum pass and the selection kernels.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    pass1 = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps   # stats + merge kernels
    pass2 = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps   # column-sum kernel
    select = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps  # page + cluster + top-k
    log(f"per step: {ms_step * 1e3:.1f} us wall; events: score pass1+merge {pass1 * 1e3:.1f} us, "
        f"pass2 {pass2 * 1e3:.1f} us, select {select * 1e3:.1f} us")

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
            "traffic": None,
            "alg_bytes_per_launch": alg_bytes,
            "kernel_us": dom_ms * 1e3,
            "mfma_frac": flops / (dom_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "step_event_us": {"score_pass1_merge": pass1 * 1e3, "score_pass2": pass2 * 1e3,
                              "page_cluster_topk": select * 1e3},
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
