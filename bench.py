#!/usr/bin/env python3
"""Benchmark: sparse decode tokens/s and effective HBM bandwidth on one MI355X.

Workload (default): one decode layer shaped like the replay study's model
(32 q / 4 KV heads, head_dim 128, bf16, 16-token pages) at 29,504 cached tokens
with a 4096-token budget (top 256 pages), envelope scoring.  One step = chunk
scoring + per-KV-head top-k + split-K sparse attention + merge for the whole
batch; chunk metadata is built once before timing (it is amortised over 16
decode steps per page in a live loop) and its build time is reported apart.
Inputs are synthetic (seeded, see block_sparse_attention_chunk_amd/synth.py)
and resident in HBM before the timed region.  To keep the 256 MB last-level
cache from serving the reads, steps rotate over replicas of the cache and
metadata whose total exceeds 1 GiB.

Prints one JSON line.  --gpus N > 1 is refused (one GPU per box).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--budget", type=int, default=4096, help="attended tokens per (sequence, KV head)")
    ap.add_argument("--scoring", choices=["envelope", "centroid"], default="envelope")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--seq-len", type=int, default=29504)
    ap.add_argument("--replicas-gib", type=float, default=1.0, help="rotate replicas until this much is touched")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extra", action="store_true", help="also time the batched and prefill workloads")
    return ap.parse_args()


class Step:
    """Device buffers and the hot path of one decode step."""

    def __init__(self, case, budget_tokens, scoring, replicas, dev):
        import torch
        from block_sparse_attention_chunk_amd import ops
        self.ops, self.torch = ops, torch
        self.case = case
        self.kind = ops.BSA_ENVELOPE if scoring == "envelope" else ops.BSA_CENTROID
        self.k_pages = budget_tokens // case.page_size
        self.budget = ops.Budget.topk(self.k_pages)
        base_k, base_v = ops.upload(case.k, dev), ops.upload(case.v, dev)
        self.q = ops.upload(case.q, dev)
        bt, sl = ops.upload(case.block_table, dev), ops.upload(case.seq_lens, dev)
        which = ops.BSA_META_ENVELOPE if self.kind == ops.BSA_ENVELOPE else ops.BSA_META_CENTROID
        self.reps = []
        for r in range(replicas):
            k = base_k if r == 0 else base_k.clone()
            v = base_v if r == 0 else base_v.clone()
            kv = ops.KVCache(k, v, sl, case.page_size, bt)
            meta = ops.build_chunk_meta(kv, which=which)
            self.reps.append((kv, meta))
        kv0 = self.reps[0][0]
        self.max_sel = self.budget.max_selected(kv0.max_pages)
        self.scores = torch.empty((case.batch, case.num_kv_heads, kv0.max_pages), dtype=torch.float32, device=dev)
        self.sel = torch.empty((case.batch, case.num_kv_heads, self.max_sel), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((case.batch, case.num_kv_heads), dtype=torch.int32, device=dev)
        self.out = torch.empty((case.batch, case.num_q_heads, case.head_dim), dtype=torch.float32, device=dev)
        need = ops.decode_workspace_bytes(kv0, case.num_q_heads, self.max_sel)
        self.ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        self.splits = ops.decode_num_splits(kv0, case.num_q_heads, self.max_sel)
        self.meta_which = which

    def run(self, i, ev=None):
        ops = self.ops
        kv, meta = self.reps[i % len(self.reps)]
        ops.score_chunks(self.q, kv, meta, self.kind, out=self.scores)
        ops.select_topk(self.scores, kv, self.budget, max_sel=self.max_sel, sel_idx=self.sel, sel_count=self.cnt)
        if ev is not None:
            ev[0].record()
        ops.sparse_attn_decode(self.q, kv, self.sel, self.cnt, out=self.out, workspace=self.ws)
        if ev is not None:
            ev[1].record()

    def dense(self, i):
        kv, _ = self.reps[i % len(self.reps)]
        self.ops.sparse_attn_decode(self.q, kv, None, None, out=self.out, workspace=self._dense_ws(kv))

    def _dense_ws(self, kv):
        if not hasattr(self, "_dws"):
            need = self.ops.decode_workspace_bytes(kv, self.case.num_q_heads, kv.max_pages)
            self._dws = self.torch.empty((max(need, 1),), dtype=self.torch.uint8, device=self.q.device)
        return self._dws


def bytes_per_step(case, k_pages, scoring):
    """Algorithmic bytes of one step: metadata read + selected K/V + q in + out."""
    D, H, Hq, B = case.head_dim, case.num_kv_heads, case.num_q_heads, case.batch
    n_pages = int(np.sum((case.seq_lens + case.page_size - 1) // case.page_size))
    meta_per_chunk = 2 * D * 2 if scoring == "envelope" else D * 4
    meta = n_pages * H * meta_per_chunk
    sel_tokens = 0
    for b in range(B):
        L = int(case.seq_lens[b])
        sel_tokens += min(k_pages * case.page_size, L)
    kvb = sel_tokens * H * D * 2 * 2
    qo = B * Hq * D * (2 + 4)
    return meta, kvb, qo


def time_loop(fn, steps, warmup, torch):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_baseline(case, k_pages, scoring, seconds):
    """The fp64 oracle on the host cores, same inputs and stages (score + select + attention)."""
    import oracle
    oc = oracle.PagedCache(case.k, case.v, case.block_table, case.seq_lens, case.page_size, case.num_kv_heads,
                           case.head_dim)
    meta = oracle.chunk_meta(oc)
    kind = oracle.ENVELOPE if scoring == "envelope" else oracle.CENTROID
    n = case.n_chunks()
    steps, t0 = 0, time.perf_counter()
    while True:
        _, sc, _ = oracle.score_decode(case.q, oc, meta, kind)
        sel, cnt = oracle.select(np.nan_to_num(sc, nan=-np.inf), n, oracle.TOPK, top_k=k_pages, max_sel=k_pages)
        oracle.decode_attn(case.q, oc, sel, cnt)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": case.batch * steps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full decode steps of the benchmarked workload (score + select + attention) in "
                      f"{el:.1f} s, fp64, OpenMP {threads} threads"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    from block_sparse_attention_chunk_amd import ops, synth
    dev = torch.device("cuda:0")
    if a.batch == 1:
        case = synth.replay_decode(seq_len=a.seq_len)
    else:
        case = synth.replay_decode(seq_len=a.seq_len, batch=a.batch)
    k_pages = a.budget // case.page_size
    kv_bytes = (case.k.nbytes + case.v.nbytes)
    replicas = max(1, math.ceil(a.replicas_gib * 2 ** 30 / kv_bytes))
    st = Step(case, a.budget, a.scoring, replicas, dev)
    torch.cuda.synchronize()

    # metadata build, timed apart
    kv0 = st.reps[0][0]
    t_meta = time_loop(lambda i: ops.build_chunk_meta(st.reps[i % replicas][0], which=st.meta_which,
                                                      meta=st.reps[i % replicas][1]), 20, 3, torch)

    # the timed region: K full steps
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for i in range(a.warmup):
        st.run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        st.run(a.warmup + i, evs[i])
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / a.steps
    t_attn = float(np.mean([s.elapsed_time(e) for s, e in evs])) * 1e-3
    t_dense = time_loop(st.dense, max(20, a.steps // 4), 5, torch)

    meta_b, kv_b, qo_b = bytes_per_step(case, k_pages, a.scoring)
    step_bytes = meta_b + kv_b + qo_b
    tok_s = case.batch / t_step
    eff_gbs = step_bytes / t_step / 1e9
    attn_gbs = kv_b / t_attn / 1e9
    n_pages = int(np.sum((case.seq_lens + 15) // 16))
    dense_kv = int(np.sum(case.seq_lens)) * case.num_kv_heads * case.head_dim * 4
    res = {
        "metric": "sparse decode tokens/s + effective HBM GB/s (% of peak) at 32K ctx, budget 4096",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values, planted needle pages, 4 outlier channels x8)",
        "config": {"workload": f"replay-shaped decode layer, {a.scoring} scoring, top-{k_pages} pages "
                               f"(budget {k_pages * 16} tokens) of {n_pages} 16-token pages",
                   "batch": case.batch, "seq_len": int(case.seq_lens[0]), "q_heads": case.num_q_heads,
                   "kv_heads": case.num_kv_heads, "head_dim": case.head_dim, "page_size": case.page_size,
                   "budget_tokens": a.budget, "scoring": a.scoring, "splits": st.splits,
                   "cache_replicas": replicas},
        "effective_hbm_gbs": eff_gbs,
        "effective_hbm_frac": eff_gbs / HBM_PEAK_GBS,
        "bytes_per_step": {"metadata": meta_b, "selected_kv": kv_b, "q_out": qo_b},
        "meta_build_us": t_meta * 1e6,
        "dense_decode_us": t_dense * 1e6,
        "sparse_attn_us": t_attn * 1e6,
        "speedup_vs_dense_attention": t_dense / t_attn,
        "speedup_vs_dense_step": t_dense / t_step,
        "roofline": {"bound": "hbm", "kernel": "bsa_sparse_attn_decode (split-K kernel + merge)",
                     "achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS,
                     "traffic": None},
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, k_pages, a.scoring, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
