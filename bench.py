#!/usr/bin/env python3
"""Benchmark of the CSA / HCA attention step on one MI355X.

Default workload (csa_decode_64k): 8 sequences at 64K context, m = 4 (16,384
compressed entries each), 128 query heads x 512, indexer 64 heads x 128, top-1024,
128-token window.  One step = one fused csa_decode call: lightning indexer over
every visible index key, causal top-1024, sparse MQA over the selected entries plus
the window (RMSNorm folded in).  Other workloads (--workload):
  hca_decode_1m      4 sequences at 1M context, m = 128 (8,192 entries), dense MQA
  csa_decode_1m_fp4  1 sequence at 1M context (262,144 entries), MXFP4 indexer
                     (the per-step query quantisation included), top-1024, MQA
  csa_prefill_4k     4,096 new queries on 61,440 prior tokens: compression of the new
                     blocks (KV and index keys), indexer + top-1024 per query, MQA
  csa_decode_1m_fp4_rescored
                     csa_decode_1m_fp4 with the labelled selector variant: MXFP4
                     prefilter of 8,192 candidates, bf16 rescoring, top-1024
  csa_decode_64k_fp8 csa_decode_64k with the compressed entries and window rows in
                     FP8 E4M3
  csa_prefill_4k_fp8 csa_prefill_4k with an FP8 E4M3 cache: the new entries are
                     compressed, then quantised into it

Inputs are seeded synthetic data resident in HBM before timing starts.  Decode
steps cycle through replicas of every cache so that the 256 MB Infinity Cache
cannot serve one step from the previous (cold-cache numbers; a warm-cache figure
with a single replica is reported too).  The timed steps are exactly --steps steps
replayed from one HIP graph, bracketed by synchronisations; the same graph is then
replayed again (50 times, or fewer when that would exceed ~30 s) to give the
median and the 10th / 90th percentiles of the time per step.

Prints ONE JSON line.  `roofline` is for the kernel that takes the largest share of
the step; its duration is measured live from HIP events that the runtime stamps with
each dispatch's own start and end (the library's timing mode, eager launches on the
kernel's stream), and `profile_avg_us` / `frac_profile` give the same figures from
the committed rocprofv3 summary of this workload (profiles/kernels_<workload>.txt).
`traffic` comes from the committed FETCH_SIZE / WRITE_SIZE counter summary when the
kernel's sources are unchanged since it was taken.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload, on one thread and as independent
single-thread processes on the host's cores; it runs before the GPU is touched.
"""
import argparse
import json
import multiprocessing
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp4": 10100.0}
WORKLOADS = ["csa_decode_64k", "hca_decode_1m", "csa_decode_1m_fp4", "csa_prefill_4k", "csa_decode_1m_fp4_rescored",
             "csa_decode_64k_fp8", "csa_prefill_4k_fp8"]
CALIB_BYTES = 256 << 20
CPU_SECONDS = 10.0        # oracle work per CPU measurement (single thread, then every core)
CPU_PROCS_MAX = 16        # the host share of one GPU
STAT_SAMPLES = 50
STAT_BUDGET_S = 30.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="csa_decode_64k", choices=WORKLOADS)
    p.add_argument("--replicas", type=int, default=16, help="cache replicas cycled by decode steps")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--pmc-pass", action="store_true",
                   help="counter-collection pass: a few eager steps plus one calibration copy of "
                        "%d MiB, no timing output" % (CALIB_BYTES >> 20))
    return p.parse_args()


# ------------------------------------------------------------------------------------
class Step:
    """One workload: host inputs (__init__), their GPU copies and a step launcher
    (setup / launch), per-kernel algorithmic work (bytes for HBM-bound kernels, flops
    for MFMA-bound ones) per launch, and the oracle's unit of work for the CPU
    baseline (cpu_prepare / cpu_unit: one token's worth unless cpu_tokens says)."""
    name = ""
    metric = ""
    dtype = "bf16"
    tokens = 1
    replicas = 1
    data = "synthetic (seeded N(0,1) caches, token streams and queries; U[0,1) indexer head weights)"
    cpu_sample = ""

    def setup(self, dev):
        raise NotImplementedError

    def launch(self, i):
        raise NotImplementedError

    def algorithmic(self, kernel):
        return None

    def cpu_prepare(self):
        pass

    def cpu_unit(self, i):
        raise NotImplementedError

    def cpu_tokens(self, units, secs, procs):
        """tokens/s from `units` oracle units in `secs` on `procs` processes."""
        return units / secs


def _torch():
    import torch
    return torch


def to_dev(x, dev):
    torch = _torch()
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(x).to(dev)


def i32(x, dev):
    torch = _torch()
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(dev)


class CsaDecode64k(Step):
    name = "csa_decode_64k"
    metric = "CSA decode tokens/s at 64K context (one layer, 8 sequences)"
    fp8 = False   # the compressed entries and window rows as FP8 E4M3 codes

    def __init__(self, R):
        from long_context_compressed_04_amd import workloads as W
        self.B, self.T, self.m, self.H, self.d, self.HI, self.dI, self.k, self.w = 8, 65536, 4, 128, 512, 64, 128, \
            1024, 128
        self.N = self.T // self.m
        self.tokens = self.B
        self.replicas = R
        c = W.csa_decode(0, B=self.B, T=self.T, m=self.m, H=self.H, d=self.d, HI=self.HI, dI=self.dI, k=self.k,
                         window=self.w)
        if self.fp8:   # codes drawn after the other tensors (the bf16 workload's draws are unchanged)
            rng = W.rng_for(1)
            c["kv"] = W.fp8_cache_codes(rng, c["kv"].shape)
            c["kv_raw"] = W.fp8_cache_codes(rng, c["kv_raw"].shape)
        self.c = c
        self.config = {"workload": self.name, "batch": self.B, "context": self.T, "compress_ratio": self.m,
                       "entries": self.N, "heads": self.H, "head_dim": self.d, "idx_heads": self.HI,
                       "idx_dim": self.dI, "topk": self.k, "window": self.w, "cache_replicas": R}
        if self.fp8:
            self.config["cache_dtype"] = "fp8_e4m3"
        B, N, k, w, d, H, HI, dI = self.B, self.N, self.k, self.w, self.d, self.H, self.HI, self.dI
        self.row_bytes = d * (1 if self.fp8 else 2)
        self.step_bytes = B * N * dI * 2 + B * (k + w) * self.row_bytes + 2 * B * H * d * 2 + B * HI * dI * 2 \
            + B * HI * 4 + B * k * 4
        self.step_flops = 2.0 * B * N * HI * dI + 4.0 * B * H * d * (k + w)

    def setup(self, dev):
        from long_context_compressed_04_amd import csa
        c, R = self.c, self.replicas
        base = dict(q=to_dev(c["q"][:, None], dev), kv=to_dev(c["kv"], dev), kv_raw=to_dev(c["kv_raw"], dev),
                    qI=to_dev(c["qI"][:, None], dev), w=to_dev(c["w"][:, None], dev), kI=to_dev(c["kI"], dev))
        rb, qp, ne = i32(c["raw_base"], dev), i32(c["q_pos"][:, None], dev), i32(c["n_entries"], dev)
        reps = [base] + [{key: t.clone() for key, t in base.items()} for _ in range(R - 1)]
        self.decs = [csa.Decoder(r["q"], r["kv"], r["kv_raw"], rb, qp, r["qI"], r["w"], r["kI"], ne, m=self.m,
                                 topk=self.k, window=self.w) for r in reps]

    def launch(self, i):
        self.decs[i % self.replicas]()

    def algorithmic(self, kernel):
        B, N, k, w, d, H, HI, dI = self.B, self.N, self.k, self.w, self.d, self.H, self.HI, self.dI
        if kernel == "index_scores_bf16":
            return "hbm", B * N * dI * 2 + B * HI * dI * 2 + B * HI * 4 + B * N * 4
        if kernel == "topk":
            return "hbm", B * N * 4 + B * k * 4
        if kernel.startswith("mqa_bf16") or kernel.startswith("mqa_f8"):
            return "hbm", B * (k + w) * self.row_bytes + 2 * B * H * d * 2 + B * k * 4
        return None

    def cpu_prepare(self):
        import oracle
        from long_context_compressed_04_amd import workloads as W
        c = self.c
        rows = (lambda x: oracle.fp8_dequantize(x)) if self.fp8 else W.value
        self.vals = [(W.value(c["q"][b]), rows(c["kv"][b]), W.value(c["qI"][b]), c["w"][b], W.value(c["kI"][b]),
                      rows(c["kv_raw"][b]), int(c["raw_base"][b]), int(c["q_pos"][b])) for b in range(self.B)]
        self.cpu_sample = ("whole decode steps of one sequence each (indexer over 16,384 keys, top-1024, MQA over "
                           "1,152 rows x 128 heads%s), fp64, sequences in turn"
                           % (", FP8 rows dequantised" if self.fp8 else ""))

    def cpu_unit(self, i):
        import oracle
        q, kv, qI, w, kI, raw, rb, t = self.vals[i % len(self.vals)]
        oracle.csa_decode_query(q, kv, self.c["N"], self.m, qI, w, kI, self.k, raw, rb, t, self.w, self.c["scale"],
                                self.c["eps"])


class CsaDecode64kFp8(CsaDecode64k):
    name = "csa_decode_64k_fp8"
    metric = "CSA decode tokens/s at 64K context with an FP8 E4M3 KV cache (one layer, 8 sequences)"
    dtype = "bf16+fp8_e4m3_kv"
    fp8 = True
    data = ("synthetic (seeded FP8 E4M3 cache codes of unit-scale values; N(0,1) queries and index keys; U[0,1) "
            "indexer head weights)")


class HcaDecode1m(Step):
    name = "hca_decode_1m"
    metric = "HCA decode tokens/s at 1M context (one layer, 4 sequences)"

    def __init__(self, R):
        from long_context_compressed_04_amd import workloads as W
        c = W.cfg3()
        self.c = c
        self.B, self.N, self.m, self.H, self.d, self.w = 4, c["N"], 128, 128, 512, 128
        self.tokens = self.B
        self.replicas = R
        self.config = {"workload": self.name, "batch": self.B, "context": 1 << 20, "compress_ratio": self.m,
                       "entries": self.N, "heads": self.H, "head_dim": self.d, "window": self.w,
                       "cache_replicas": R}
        B, N, w, d, H = self.B, self.N, self.w, self.d, self.H
        self.step_bytes = B * (N + w) * d * 2 + 2 * B * H * d * 2
        self.step_flops = 4.0 * B * H * d * (N + w)

    def setup(self, dev):
        import ctypes
        torch = _torch()
        from long_context_compressed_04_amd import csa
        c, R = self.c, self.replicas
        base = dict(q=to_dev(c["q"][:, None], dev), kv=to_dev(c["kv"], dev), kv_raw=to_dev(c["kv_raw"], dev))
        self.rb, self.qp, self.ne = i32(c["raw_base"], dev), i32(c["q_pos"][:, None], dev), i32(c["n_entries"], dev)
        self.reps = [base] + [{key: t.clone() for key, t in base.items()} for _ in range(R - 1)]
        self.out = torch.empty_like(base["q"])
        self.lse = torch.empty(base["q"].shape[:3], dtype=torch.float32, device=dev)
        d = csa._mqa_desc(base["q"], base["kv"], base["kv_raw"], m=self.m, n_max=self.N, window=self.w)
        self.ws = torch.zeros(max(1, csa.lib().csa_mqa_workspace_size(ctypes.byref(d), 1)), dtype=torch.uint8,
                              device=dev)
        self.csa = csa

    def launch(self, i):
        r = self.reps[i % self.replicas]
        self.csa.hca_dense_mqa(r["q"], r["kv"], self.ne, r["kv_raw"], self.rb, self.qp, m=self.m, window=self.w,
                               workspace=self.ws, out=self.out, lse=self.lse)

    def algorithmic(self, kernel):
        if kernel.startswith("mqa_bf16"):
            return "hbm", self.step_bytes
        return None

    def cpu_prepare(self):
        from long_context_compressed_04_amd import workloads as W
        c = self.c
        self.vals = [(W.value(c["q"][b]), W.value(c["kv"][b]), W.value(c["kv_raw"][b]), int(c["raw_base"][b]),
                      int(c["q_pos"][b])) for b in range(self.B)]
        self.cpu_sample = "decode steps of one sequence each (dense MQA over 8,320 rows x 128 heads), fp64"

    def cpu_unit(self, i):
        import oracle
        q, kv, raw, rb, t = self.vals[i % len(self.vals)]
        oracle.dense_mqa(q, kv, self.N, self.m, raw, rb, t, self.w, self.c["scale"], self.c["eps"])


class CsaDecode1mFp4(Step):
    name = "csa_decode_1m_fp4"
    metric = "CSA decode tokens/s at 1M context with the MXFP4 indexer (one layer, 1 sequence)"
    dtype = "bf16+mxfp4_indexer"

    def __init__(self, R):
        from long_context_compressed_04_amd import workloads as W
        c = W.cfg4()
        self.c = c
        self.N, self.m, self.H, self.d, self.HI, self.dI, self.k, self.w = c["N"], 4, 128, 512, 64, 128, 1024, 128
        self.tokens = 1
        self.replicas = R
        self.config = {"workload": self.name, "batch": 1, "context": 1 << 20, "compress_ratio": self.m,
                       "entries": self.N, "heads": self.H, "head_dim": self.d, "idx_heads": self.HI,
                       "idx_dim": self.dI, "idx_dtype": "mxfp4", "topk": self.k, "window": self.w,
                       "cache_replicas": R}
        N, k, w, d, H, HI, dI = self.N, self.k, self.w, self.d, self.H, self.HI, self.dI
        self.key_bytes = N * (dI // 2 + dI // 32)
        self.step_bytes = self.key_bytes + (k + w) * d * 2 + 2 * H * d * 2 + HI * dI * 2 + HI * 4 + k * 4
        self.step_flops = 2.0 * N * HI * dI + 4.0 * H * d * (k + w)

    def setup(self, dev):
        from long_context_compressed_04_amd import csa
        c, R = self.c, self.replicas
        self.csa = csa
        qI = to_dev(c["qI"][:, None], dev)
        kI = to_dev(c["kI"], dev)
        base = dict(q=to_dev(c["q"][:, None], dev), kv=to_dev(c["kv"], dev), kv_raw=to_dev(c["kv_raw"], dev), qI=qI)
        # index keys are quantised once, when the cache is written
        kc, ks = csa.mxfp4_quantize(kI)
        base["kc"], base["ks"] = kc, ks
        del kI
        rb, qp, ne = i32(c["raw_base"], dev), i32(c["q_pos"][:, None], dev), i32(c["n_entries"], dev)
        w = to_dev(c["w"][:, None], dev)
        reps = [base] + [{key: t.clone() for key, t in base.items()} for _ in range(R - 1)]
        self.reps = reps
        # the fp32 indexer queries are quantised inside each step's indexer launch
        self.decs = [csa.Decoder(r["q"], r["kv"], r["kv_raw"], rb, qp, r["qI"], w, r["kc"], ne, m=self.m,
                                 topk=self.k, window=self.w, k_scale=r["ks"]) for r in reps]

    def launch(self, i):
        self.decs[i % self.replicas]()

    def algorithmic(self, kernel):
        N, k, w, d, H, HI, dI = self.N, self.k, self.w, self.d, self.H, self.HI, self.dI
        if kernel == "index_scores_mxfp4":
            return "hbm", self.key_bytes + HI * (dI // 2 + dI // 32) + HI * 4 + N * 4
        if kernel == "topk":
            return "hbm", N * 4 + k * 4
        if kernel.startswith("mqa_bf16"):
            return "hbm", (k + w) * d * 2 + 2 * H * d * 2 + k * 4
        return None

    def cpu_prepare(self):
        import oracle
        from long_context_compressed_04_amd import workloads as W
        c = self.c
        self.q, self.kv, self.raw = W.value(c["q"][0]), W.value(c["kv"][0]), W.value(c["kv_raw"][0])
        kc, ksc = oracle.mxfp4_quantize(c["kI"][0])
        self.k_deq = oracle.mxfp4_dequantize(kc, ksc)      # at cache write, not per step
        self.cpu_sample = ("whole decode steps (query quantisation, indexer over 262,144 dequantised keys, "
                           "top-1024, MQA over 1,152 rows x 128 heads), fp64")

    def cpu_unit(self, i):
        import oracle
        c = self.c
        q_deq = oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(c["qI"][0]))
        oracle.csa_decode_query(self.q, self.kv, self.N, self.m, q_deq, c["w"][0], self.k_deq, self.k, self.raw,
                                int(c["raw_base"][0]), int(c["q_pos"][0]), self.w, c["scale"], c["eps"])


class CsaDecode1mFp4Rescored(CsaDecode1mFp4):
    """The labelled selector variant on the 1M FP4 workload: the MXFP4 scores pick 8,192
    candidates, bf16 copies of q^I and K^I rescore them, the top-1024 rescored
    candidates feed the MQA (two library calls per step)."""
    name = "csa_decode_1m_fp4_rescored"
    metric = ("CSA decode tokens/s at 1M context, MXFP4 prefilter + bf16 rescoring selector "
              "(one layer, 1 sequence)")
    dtype = "bf16+mxfp4_prefilter"
    cand = 8192

    def __init__(self, R):
        super().__init__(R)
        self.config.update(workload=self.name, selector="mxfp4 prefilter + bf16 rescoring", candidates=self.cand)
        self.step_bytes += self.cand * 4 + self.cand * self.dI * 2

    def setup(self, dev):
        import ctypes
        super().setup(dev)
        torch = _torch()
        from long_context_compressed_04_amd import workloads as W
        c = self.c
        q16 = to_dev(W.store(c["qI"][:, None], "bf16"), dev)
        k16 = to_dev(W.store(c["kI"], "bf16"), dev)
        for j, r in enumerate(self.reps):
            r["q16"] = q16 if j == 0 else q16.clone()
            r["k16"] = k16 if j == 0 else k16.clone()
        self.w_dev = to_dev(c["w"][:, None], dev)
        self.rb, self.qp, self.ne = (i32(c["raw_base"], dev), i32(c["q_pos"][:, None], dev),
                                     i32(c["n_entries"], dev))
        r0 = self.reps[0]
        d = self.csa._index_desc(r0["qI"], r0["kc"], 4, self.k, None, *self.csa._index_dtype(r0["qI"], r0["kc"]))
        self.ws_i = torch.zeros(self.csa.lib().csa_index_rescored_workspace_size(ctypes.byref(d), self.cand),
                                dtype=torch.uint8, device=dev)
        dm = self.csa._mqa_desc(r0["q"], r0["kv"], r0["kv_raw"], topk=self.k, window=self.w)
        self.ws_m = torch.zeros(max(1, self.csa.lib().csa_mqa_workspace_size(ctypes.byref(dm), 0)),
                                dtype=torch.uint8, device=dev)
        self.idx = torch.empty((1, 1, self.k), dtype=torch.int32, device=dev)
        self.isc = torch.empty((1, 1, self.k), dtype=torch.float32, device=dev)
        self.out = torch.empty_like(r0["q"])
        self.lse = torch.empty(r0["q"].shape[:3], dtype=torch.float32, device=dev)

    def launch(self, i):
        r = self.reps[i % self.replicas]
        csa = self.csa
        csa.index_topk_rescored(r["qI"], None, r["q16"], self.w_dev, r["kc"], r["ks"], r["k16"], self.ne, self.qp,
                                m=self.m, topk=self.k, cand=self.cand, workspace=self.ws_i, out_idx=self.idx,
                                out_score=self.isc)
        csa.sparse_mqa(r["q"], r["kv"], self.idx, r["kv_raw"], self.rb, self.qp, window=self.w, workspace=self.ws_m,
                       out=self.out, lse=self.lse)

    def algorithmic(self, kernel):
        if kernel == "index_rescore_bf16":
            return "hbm", self.cand * (4 + self.dI * 2) + self.HI * self.dI * 2 + self.cand * 4
        if kernel == "topk":   # the prefilter's and the final selection's reads and writes
            return "hbm", self.N * 4 + self.cand * 4 + self.cand * 4 + self.k * 4
        return super().algorithmic(kernel)

    def cpu_prepare(self):
        from long_context_compressed_04_amd import workloads as W
        super().cpu_prepare()
        c = self.c
        self.k16 = W.value(W.store(c["kI"][0], "bf16"))
        self.q16 = W.value(W.store(c["qI"][0], "bf16"))
        self.cpu_sample = ("whole decode steps (query quantisation, MXFP4 scores over 262,144 keys, top-8192, bf16 "
                           "rescoring, top-1024, MQA over 1,152 rows x 128 heads), fp64")

    def cpu_unit(self, i):
        import oracle
        c = self.c
        q_deq = oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(c["qI"][0]))
        idx, _, _ = oracle.index_topk_rescored(q_deq, c["w"][0], self.k_deq, self.q16, self.k16, self.N, self.cand,
                                               self.k)
        oracle.sparse_mqa(self.q, self.kv, idx, self.raw, int(c["raw_base"][0]), int(c["q_pos"][0]), self.w,
                          c["scale"], c["eps"])


class CsaPrefill4k(Step):
    name = "csa_prefill_4k"
    metric = "CSA prefill tokens/s (4,096 new queries on 61,440 prior tokens, one layer)"

    def __init__(self, R):
        from long_context_compressed_04_amd import workloads as W
        c = W.cfg5()
        self.c = c
        self.replicas = 1
        N, P, d, dI = c["N"], c["P"], c["d"], c["dI"]
        self.N, self.P, self.Q, self.H, self.d, self.HI, self.dI, self.k, self.w, self.m = \
            N, P, c["n_new"], c["H"], d, c["HI"], dI, c["k"], c["window"], c["m"]
        self.tokens = self.Q
        self.tb = c["tok_base"]
        self.config = {"workload": self.name, "batch": 1, "new_tokens": self.Q, "prior_tokens": c["T_prior"],
                       "compress_ratio": self.m, "entries": N, "heads": self.H, "head_dim": d,
                       "idx_heads": self.HI, "idx_dim": dI, "topk": self.k, "window": self.w}
        vis = np.minimum(N, (c["q_pos"].astype(np.int64) + 1) // self.m)
        self.pairs = int(vis.sum())
        sel = np.minimum(vis, self.k) + np.minimum(c["q_pos"].astype(np.int64) + 1, self.w)
        self.mqa_rows = int(sel.sum())
        R_tok = self.Q + self.m
        self.compress_bytes = {d: R_tok * d * 2 * 2 + R_tok * 4 * 2 + (N - P) * d * 2 for d in (d, dI)}
        self.step_flops = 2.0 * self.pairs * self.HI * dI + 4.0 * self.H * d * self.mqa_rows
        # compulsory: the compression's token rows, logits and new entries; every index
        # key once; q, out, q_idx, w and the selection of every query; every compressed
        # entry and raw window row at most once
        self.step_bytes = sum(self.compress_bytes.values()) + N * dI * 2 + \
            self.Q * (self.H * d * 2 * 2 + self.HI * dI * 2 + self.HI * 4 + self.k * 4) + \
            N * d * 2 + (self.Q + self.w - 1) * d * 2

    def setup(self, dev):
        import ctypes
        torch = _torch()
        from long_context_compressed_04_amd import csa
        c = self.c
        self.csa = csa
        N, P, d, dI = self.N, self.P, self.d, self.dI
        self.kv = torch.zeros((1, N, d), dtype=torch.bfloat16, device=dev)
        self.kI = torch.zeros((1, N, dI), dtype=torch.bfloat16, device=dev)
        self.kv[0, :P] = to_dev(c["kv_prior"], dev)
        self.kI[0, :P] = to_dev(c["kI_prior"], dev)
        self.A, self.Bs, self.z = to_dev(c["A"][None], dev), to_dev(c["Bs"][None], dev), to_dev(c["z"][None], dev)
        self.AI, self.BI, self.zI = to_dev(c["AI"][None], dev), to_dev(c["BI"][None], dev), to_dev(c["zI"][None], dev)
        self.q, self.qI, self.wt = to_dev(c["q"][None], dev), to_dev(c["qI"][None], dev), to_dev(c["w"][None], dev)
        self.raw = to_dev(c["kv_raw"][None], dev)
        self.q_pos = i32(c["q_pos"][None], dev)
        self.rb = i32([c["raw_base"]], dev)
        self.ne = i32([N], dev)
        di = csa._index_desc(self.qI, self.kI, self.m, self.k, None, csa.BF16)
        self.idx_ws = torch.zeros(csa.lib().csa_index_workspace_size(ctypes.byref(di)), dtype=torch.uint8,
                                  device=dev)
        dm = csa._mqa_desc(self.q, self.kv, self.raw, topk=self.k, window=self.w)
        self.mqa_ws = torch.zeros(max(1, csa.lib().csa_mqa_workspace_size(ctypes.byref(dm), 0)), dtype=torch.uint8,
                                  device=dev)
        self.idx = torch.empty((1, self.Q, self.k), dtype=torch.int32, device=dev)
        self.score = torch.empty((1, self.Q, self.k), dtype=torch.float32, device=dev)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=dev)

    def launch(self, i):
        csa = self.csa
        csa.compress(self.A, self.Bs, self.z, self.z, self.m, self.kv, tok_base=self.tb, entry_begin=self.P,
                     entry_end=self.N)
        csa.compress(self.AI, self.BI, self.zI, self.zI, self.m, self.kI, tok_base=self.tb, entry_begin=self.P,
                     entry_end=self.N)
        csa.index_topk(self.qI, self.wt, self.kI, self.ne, self.q_pos, m=self.m, topk=self.k,
                       workspace=self.idx_ws, out_idx=self.idx, out_score=self.score)
        csa.sparse_mqa(self.q, self.kv, self.idx, self.raw, self.rb, self.q_pos, window=self.w,
                       workspace=self.mqa_ws, out=self.out, lse=self.lse)

    def algorithmic(self, kernel):
        if kernel == "index_scores_bf16":
            return "mfma", 2.0 * self.pairs * self.HI * self.dI
        if kernel.startswith("mqa_bf16"):
            return "mfma", 4.0 * self.H * self.d * self.mqa_rows
        if kernel == "topk":
            return "hbm", self.pairs * 4 + self.Q * self.k * 4
        return None

    def cpu_prepare(self):
        import oracle
        from long_context_compressed_04_amd import workloads as W
        c = self.c
        t0 = time.perf_counter()
        new_kv = oracle.compress(W.value(c["A"]), W.value(c["Bs"]), c["z"], c["z"], self.m, tok_base=self.tb,
                                 entry_begin=self.P, entry_end=self.N)
        new_kI = oracle.compress(W.value(c["AI"]), W.value(c["BI"]), c["zI"], c["zI"], self.m, tok_base=self.tb,
                                 entry_begin=self.P, entry_end=self.N)
        self.t_compress = time.perf_counter() - t0
        self.keys = np.concatenate([W.value(c["kI_prior"]), new_kI])
        self.kv_all = np.concatenate([W.value(c["kv_prior"]), new_kv])
        self.raw_v = W.value(c["kv_raw"])
        self.order = list(range(0, self.Q, 128))
        self.cpu_sample = ("queries taken every 128th (indexer, top-1024, MQA), scaled to all 4,096, plus the "
                           "compression of the 1,024 new entries (KV and index keys) timed in full (%.1f s on one "
                           "thread, divided by the process count for all cores); fp64" % self.t_compress)

    def cpu_unit(self, i):
        import oracle
        from long_context_compressed_04_amd import workloads as W
        c = self.c
        qi = self.order[i % len(self.order)]
        t = int(c["q_pos"][qi])
        V = oracle.visible(t, self.N, self.m)
        scores = oracle.index_scores(W.value(c["qI"][qi]), c["w"][qi], self.keys[:V])
        idx = oracle.topk(scores, V, self.k)
        oracle.sparse_mqa(W.value(c["q"][qi]), self.kv_all, idx, self.raw_v, c["raw_base"], t, self.w, c["scale"],
                          c["eps"])

    def cpu_tokens(self, units, secs, procs):
        query_s = secs / units * procs            # seconds of one query on one thread
        return self.Q / (self.t_compress / procs + self.Q * query_s / procs)


class CsaPrefill4kFp8(CsaPrefill4k):
    """csa_prefill_4k with the compressed entries and the window rows held as FP8 E4M3
    codes: the step compresses the new entries (bf16), quantises them into the cache,
    and attends the FP8 rows (through the 8-wave kernel's normalising pre-pass)."""
    name = "csa_prefill_4k_fp8"
    metric = "CSA prefill tokens/s with an FP8 E4M3 KV cache (4,096 new queries on 61,440 prior tokens, one layer)"
    dtype = "bf16+fp8_e4m3_kv"

    def __init__(self, R):
        super().__init__(R)
        self.config["workload"] = self.name
        self.config["cache_dtype"] = "fp8_e4m3"

    def setup(self, dev):
        super().setup(dev)
        csa = self.csa
        N, P = self.N, self.P
        import ctypes
        torch = _torch()
        self.kv8 = csa.fp8_quantize(self.kv)            # the prior entries (new ones per step)
        self.raw8 = csa.fp8_quantize(self.raw)
        self.new_bf16 = self.kv[0, P:N]                  # where the step's compression lands
        self.new_codes = self.kv8[0, P:N]
        dm = csa._mqa_desc(self.q, self.kv8, self.raw8, topk=self.k, window=self.w)
        self.mqa_ws = torch.zeros(max(1, csa.lib().csa_mqa_workspace_size(ctypes.byref(dm), 0)), dtype=torch.uint8,
                                  device=dev)

    def cpu_prepare(self):
        import oracle
        super().cpu_prepare()
        # the attention reads the rows' FP8 codes at their exact values
        self.kv_all = oracle.fp8_dequantize(oracle.fp8_quantize(self.kv_all)).reshape(self.kv_all.shape)
        self.raw_v = oracle.fp8_dequantize(oracle.fp8_quantize(self.raw_v)).reshape(self.raw_v.shape)
        self.cpu_sample += "; FP8 rows dequantised"

    def launch(self, i):
        csa = self.csa
        csa.compress(self.A, self.Bs, self.z, self.z, self.m, self.kv, tok_base=self.tb, entry_begin=self.P,
                     entry_end=self.N)
        csa.fp8_quantize(self.new_bf16, self.new_codes)
        csa.compress(self.AI, self.BI, self.zI, self.zI, self.m, self.kI, tok_base=self.tb, entry_begin=self.P,
                     entry_end=self.N)
        csa.index_topk(self.qI, self.wt, self.kI, self.ne, self.q_pos, m=self.m, topk=self.k,
                       workspace=self.idx_ws, out_idx=self.idx, out_score=self.score)
        csa.sparse_mqa(self.q, self.kv8, self.idx, self.raw8, self.rb, self.q_pos, window=self.w,
                       workspace=self.mqa_ws, out=self.out, lse=self.lse)


def make(name, R):
    return {"csa_decode_64k": CsaDecode64k, "csa_decode_64k_fp8": CsaDecode64kFp8, "hca_decode_1m": HcaDecode1m,
            "csa_decode_1m_fp4": CsaDecode1mFp4, "csa_prefill_4k_fp8": CsaPrefill4kFp8,
            "csa_prefill_4k": CsaPrefill4k, "csa_decode_1m_fp4_rescored": CsaDecode1mFp4Rescored}[name](R)


# ------------------------------------------------------------------ CPU baseline
_CPU_WL = None


def _cpu_worker(start):
    """Oracle units from `start` on, until CPU_SECONDS have passed (one thread)."""
    n, t0 = 0, time.perf_counter()
    while True:
        _CPU_WL.cpu_unit(start + n)
        n += 1
        secs = time.perf_counter() - t0
        if secs >= CPU_SECONDS:
            return n, secs


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(wl):
    """The oracle as committed, on one thread, then as independent single-thread
    processes on the host's cores (forked before any GPU use)."""
    global _CPU_WL
    wl.cpu_prepare()
    _CPU_WL = wl
    n1, s1 = _cpu_worker(0)
    procs = max(1, min(CPU_PROCS_MAX, os.cpu_count() or 1))
    res = {"value": round(wl.cpu_tokens(n1, s1, 1), 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": "%d %s; one thread, %.1f s" % (n1, wl.cpu_sample, s1),
           "host_cpu": _cpu_model(), "host_logical_cpus": os.cpu_count()}
    try:
        with multiprocessing.get_context("fork").Pool(procs) as pool:
            parts = pool.map(_cpu_worker, [1000 * p for p in range(procs)])
        n_all = sum(p[0] for p in parts)
        secs = max(p[1] for p in parts)
        res["all_cores"] = {"value": round(wl.cpu_tokens(n_all, secs, procs), 4), "unit": "tokens/s",
                            "cores": procs,
                            "sample": "%d units on %d independent single-thread processes, %.1f s"
                                      % (n_all, procs, secs)}
    except Exception as e:    # the single-thread figure stands on its own
        res["all_cores"] = {"value": None, "error": repr(e)}
    return res


# ------------------------------------------------------------------ profiles
def profile_avg_us(workload, kernel):
    """Average duration of a library kernel in the committed rocprofv3 summary."""
    path = os.path.join(ROOT, "profiles", "kernels_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 3 and parts[0] == kernel:
                try:
                    return float(parts[2])
                except ValueError:
                    return None
    return None


def percentiles(samples):
    a = np.asarray(samples, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "samples": int(a.size)}


# ------------------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this implementation runs on a single MI355X and has no multi-GPU "
              "path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    steps = max(1, args.steps)
    wl = make(args.workload, max(1, args.replicas))
    cpu = None
    if not args.no_cpu_baseline and not args.pmc_pass:
        cpu = cpu_baseline(wl)          # before the GPU is initialised: the pool forks this process
        print("cpu baseline done", file=sys.stderr, flush=True)

    import torch
    from long_context_compressed_04_amd import csa
    from long_context_compressed_04_amd import profiling

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    csa.lib()
    wl.setup(dev)
    R = wl.replicas
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    if args.pmc_pass:
        for i in range(2 * R):
            wl.launch(i)
        torch.cuda.synchronize()
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print("pmc pass done: %s, %d steps, calibration copy %d bytes" % (wl.name, 2 * R, CALIB_BYTES), flush=True)
        return

    # ---- one graph of exactly `steps` steps (step i on replica i % R)
    for i in range(R):
        wl.launch(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream(dev)):
        for i in range(steps):
            wl.launch(i)
    torch.cuda.synchronize()
    for i in range(args.warmup):        # untimed warm-up steps
        wl.launch(i)
    graph.replay()                      # and one untimed replay: the first replay of a
    torch.cuda.synchronize()            # graph carries a one-time set-up cost

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    secs = e0.elapsed_time(e1) / 1e3
    ms_per_step = secs * 1e3 / steps

    # ---- the same graph again, each replay timed: the spread of the time per step
    n_stat = int(max(5, min(STAT_SAMPLES, STAT_BUDGET_S / max(secs, 1e-6))))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_stat)]
    for a, b in evs:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    per_step = [a.elapsed_time(b) / steps for a, b in evs]

    # ---- warm cache: one replica, eager launches
    n_warm = min(steps, 50)
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(n_warm):
        wl.launch(0)
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / n_warm

    # ---- every kernel of the step, timed live (dispatch-stamped HIP events)
    csa.timing_enable(True)
    n_t = max(2 * R, 4)
    for i in range(n_t):
        wl.launch(i)
    kt = csa.timing_collect()
    csa.timing_enable(False)
    per_step_us = {k: v["avg_us"] * v["launches"] / n_t for k, v in kt.items()}
    dom = max(per_step_us, key=per_step_us.get)
    kernels = {k: {"avg_us": round(v["avg_us"], 3), "launches_per_step": round(v["launches"] / n_t, 2),
                   "us_per_step": round(per_step_us[k], 3)} for k, v in kt.items()}
    alg = wl.algorithmic(dom)
    dom_us = kt[dom]["avg_us"]
    prof_us = profile_avg_us(wl.name, dom)
    roof = {"bound": None, "kernel": dom, "achieved": None, "peak": None, "unit": None, "frac": None,
            "traffic": None, "avg_launch_us": round(dom_us, 3), "frac_source": "live dispatch-stamped HIP events",
            "profile_avg_us": prof_us, "frac_profile": None}
    if alg is not None:
        bound, amount = alg
        if bound == "hbm":
            peak, unit, scale = HBM_PEAK_GBS, "GB/s", 1e9
            roof["bytes_per_launch"] = amount
        else:
            peak = MFMA_PEAK_TFLOPS["mxfp4" if "mxfp4" in dom else "bf16"]
            unit, scale = "TFLOP/s", 1e12
            roof["flops_per_launch"] = amount
        achieved = amount / (dom_us * 1e-6) / scale
        roof.update(bound=bound, achieved=round(achieved, 1), peak=peak, unit=unit, frac=round(achieved / peak, 4))
        if prof_us:
            roof["frac_profile"] = round(amount / (prof_us * 1e-6) / scale / peak, 4)
    prof = os.path.join(ROOT, "profiles", "traffic_%s.json" % wl.name)
    if os.path.exists(prof):
        with open(prof) as f:
            pj = json.load(f)
        ent = pj.get("kernels", {}).get(dom)
        if ent and ent.get("source_hash") == profiling.source_hash(dom):
            roof["traffic"] = ent["bytes_per_launch"]

    result = {
        "metric": wl.metric,
        "value": round(wl.tokens * steps / secs, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": wl.data,
        "config": dict(wl.config, graph=True),
        "ms_per_step_stats": percentiles(per_step),
        "timed_wall_s": round(t_wall, 4),
        "step_bytes": wl.step_bytes,
        "step_flops": wl.step_flops,
        "step_hbm_frac": round(wl.step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(wl.step_flops / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
        "warm_ms_per_step": round(warm_ms, 5),
        "kernels": kernels,
        "roofline": roof,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
