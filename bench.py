#!/usr/bin/env python3
"""Benchmark: CSA decode at 64K context (8 sequences x 16,384 compressed entries,
128 query heads x 512, indexer 64 x 128, top-1024, 128-token window) on one MI355X.

One step = one fused csa_decode call: lightning indexer over every visible index
key, causal top-1024, sparse MQA over the selected entries plus the window (RMSNorm
folded in).  Inputs are resident in HBM before timing starts.  Each step reads a
different replica of the caches, so that the 256 MB Infinity Cache cannot serve a
step from the previous one (cold-cache HBM numbers; a warm figure is reported too).

Prints ONE JSON line.  Also reports the dominant kernel (the indexer) against the
HBM roofline, timed live with HIP events on its own stream, and the CPU oracle's
throughput on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=16)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", type=int, default=1, help="replay the step from a HIP graph")
    return p.parse_args()


def file_hash(*paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X and has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_compressed_04_amd import csa
    from long_context_compressed_04_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    csa.lib()

    B, T, m, H, d, HI, dI, k, window = 8, 65536, 4, 128, 512, 64, 128, 1024, 128
    N = T // m
    c = W.csa_decode(0, B=B, T=T, m=m, H=H, d=d, HI=HI, dI=dI, k=k, window=window)

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    def i32(x):
        return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(dev)

    base = dict(q=to_dev(c["q"][:, None]), kv=to_dev(c["kv"]), kv_raw=to_dev(c["kv_raw"]),
                qI=to_dev(c["qI"][:, None]), w=to_dev(c["w"][:, None]), kI=to_dev(c["kI"]))
    raw_base, q_pos, n_entries = i32(c["raw_base"]), i32(c["q_pos"][:, None]), i32(c["n_entries"])
    del c
    R = max(1, args.replicas)
    reps = [base] + [{key: t.clone() for key, t in base.items()} for _ in range(R - 1)]
    decs = [csa.Decoder(r["q"], r["kv"], r["kv_raw"], raw_base, q_pos, r["qI"], r["w"], r["kI"], n_entries,
                        m=m, topk=k, window=window) for r in reps]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    def run_steps(n, replica_cycle=True):
        for i in range(n):
            decs[i % R if replica_cycle else 0]()

    # ---- graph capture of R consecutive steps (one per replica)
    graph = None
    if args.graph:
        run_steps(R)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=torch.cuda.Stream(dev)):
            run_steps(R)
        torch.cuda.synchronize()

    def timed(n_steps, replica_cycle=True):
        if graph is not None and replica_cycle:
            reps_n = max(1, n_steps // R)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps_n):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1e3, reps_n * R
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_steps(n_steps, replica_cycle)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3, n_steps

    # warmup, then the timed region
    if graph is not None:
        for _ in range(max(1, args.warmup // R)):
            graph.replay()
    else:
        run_steps(args.warmup)
    torch.cuda.synchronize()
    secs, steps = timed(args.steps)
    ms_per_step = secs * 1e3 / steps
    tok_s = B * steps / secs

    # warm-cache figure (same replica every step, eager launches)
    warm_secs, warm_steps = timed(min(args.steps, 100), replica_cycle=False)
    warm_ms = warm_secs * 1e3 / warm_steps

    # ---- compulsory bytes of one step (cold): every visible index key, the selected
    # entries and window rows, q, q_idx, w, the output
    kv_row, key_row = d * 2, dI * 2
    step_bytes = (B * N * key_row + B * (k + window) * kv_row + B * H * d * 2 * 2 + B * HI * dI * 2 + B * HI * 4
                  + B * k * 4)
    step_flops = 2.0 * B * N * HI * dI + 4.0 * B * H * d * (k + window)

    # ---- dominant kernel: the indexer, timed per launch with HIP events on its stream
    ne_bytes = B * N * key_row + B * HI * dI * 2 + B * HI * 4 + B * N * 4
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R * 4)]
    scores_out = [torch.empty((B, 1, N), dtype=torch.float32, device=dev) for _ in range(2)]
    for i in range(R):
        r = reps[i]
        csa.index_scores(r["qI"], r["w"], r["kI"], n_entries, q_pos, m=m, n_max=N)
    torch.cuda.synchronize()
    durs = []
    lib = csa.lib()
    import ctypes
    desc = csa.IndexDesc(B, 1, HI, dI, m, k, N, N, csa.BF16)
    for j, (a, b_) in enumerate(ev):
        r = reps[j % R]
        a.record(stream)
        st = lib.csa_index_scores(ctypes.byref(desc), r["qI"].data_ptr(), None, r["w"].data_ptr(),
                                  r["kI"].data_ptr(), None, n_entries.data_ptr(), q_pos.data_ptr(),
                                  scores_out[j % 2].data_ptr(), stream.cuda_stream)
        assert st == 0
        b_.record(stream)
    torch.cuda.synchronize()
    durs = [a.elapsed_time(b_) * 1e-3 for a, b_ in ev]
    idx_s = float(np.mean(durs))
    achieved = ne_bytes / idx_s / 1e9

    traffic = None
    prof = os.path.join(ROOT, "profiles", "index_scores_bf16_csa_decode_64k_traffic.json")
    if os.path.exists(prof):
        with open(prof) as f:
            pj = json.load(f)
        if pj.get("source_hash") == file_hash("long_context_compressed_04_amd/csrc/indexer.hip"):
            traffic = pj.get("bytes_per_launch")

    result = {
        "metric": "CSA decode tokens/s at 64K context (one layer, 8 sequences)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) caches and queries, U[0,1) indexer head weights)",
        "config": {"workload": "csa_decode_64k", "batch": B, "context": T, "compress_ratio": m,
                   "entries": N, "heads": H, "head_dim": d, "idx_heads": HI, "idx_dim": dI, "topk": k,
                   "window": window, "cache_replicas": R, "graph": bool(graph is not None)},
        "step_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_bytes": step_bytes,
        "step_flops": step_flops,
        "warm_ms_per_step": round(warm_ms, 5),
        "roofline": {"bound": "hbm", "kernel": "index_scores_mfma (bf16)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": ne_bytes, "avg_launch_us": round(idx_s * 1e6, 3)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(B, T, m, H, d, HI, dI, k, window)
    print(json.dumps(result), flush=True)


def cpu_baseline(B, T, m, H, d, HI, dI, k, window):
    """The oracle (single thread, fp64) on the same workload: all sequences of one step."""
    import oracle
    from long_context_compressed_04_amd import workloads as W
    c = W.csa_decode(0, B=B, T=T, m=m, H=H, d=d, HI=HI, dI=dI, k=k, window=window)
    seqs = list(range(B))
    vals = [(W.value(c["q"][b]), W.value(c["kv"][b]), W.value(c["qI"][b]), c["w"][b], W.value(c["kI"][b]),
             W.value(c["kv_raw"][b])) for b in seqs]
    t0 = time.perf_counter()
    for b, (q, kv, qI, w, kI, raw) in zip(seqs, vals):
        oracle.csa_decode_query(q, kv, c["N"], m, qI, w, kI, k, raw, int(c["raw_base"][b]), int(c["q_pos"][b]),
                                window, c["scale"], c["eps"])
    secs = time.perf_counter() - t0
    return {"value": round(len(seqs) / secs, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "one full decode step of all %d sequences (indexer over 16,384 keys, top-1024, "
                      "MQA over 1,152 rows x 128 heads), fp64, single thread, %.1f s" % (len(seqs), secs)}


if __name__ == "__main__":
    main()
