#!/usr/bin/env python3
"""Benchmark: sparse decode tokens/s and effective HBM bandwidth on one MI355X.

Headline workload: one decode layer shaped like the replay study's model
(32 q / 4 KV heads, head_dim 128, bf16, 16-token pages) at 29,504 cached tokens
with a 4096-token budget (top 256 of 1,844 pages), envelope scoring, one
sequence.  One step = chunk scoring + per-KV-head top-k + split-K sparse
attention + split merge for the whole batch, run as the library's decode step:
bsa_score_chunks then bsa_select_attn_decode (selection fused into the
attention kernel).  The unfused sequence (bsa_select_topk then
bsa_sparse_attn_decode) is timed beside it.  Chunk metadata is built once
before timing (in a live loop a page's metadata is written once per 16 decode
steps) and its build time is reported apart.  Per-kernel figures (the fused
kernel, the decode kernel and the merge alone) come from HIP events around
graph replays of that launch alone on its stream (the split partials are left
in the workspace and merged by a separate call).

Inputs are synthetic and seeded (block_sparse_attention_chunk_amd/synth.py)
and resident in HBM before the timed region.  Steps rotate over replicas of
the cache and metadata whose total exceeds 1 GiB, so the 256 MB last-level
cache cannot serve the reads.  Each step is captured once in a HIP graph and
replayed, so host dispatch is not in the measurement.

Extra records in the same JSON line: the same layer with 16 sequences at
32,768 tokens; a 64 q / 8 KV-head batch of 16 x 32,768 tokens at ratio 1/8
(4096 tokens per sequence and head); the 131,072-token router prefill (28 q /
4 KV heads, k = 32, rho = 2) with its MFMA utilisation, and the same router
at 32,768 and 65,536 tokens; a 48-layer decode step (48 replay-shaped layers
with their own caches, one HIP graph) at 1 and 16 sequences; with --extra
also every budget against the dense kernel: top-256 / top-512 pages on the
29,504-token layer with both scorings, token budgets 4096 / 8192 / 16384 over
variable chunks, and the seven ratios of the 8K-32K batched workload with
both scorings.

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
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--budget", type=int, default=4096, help="attended tokens per (sequence, KV head)")
    ap.add_argument("--scoring", choices=["envelope", "centroid"], default="envelope")
    ap.add_argument("--replicas-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-batched", action="store_true", help="skip the batched extra records")
    ap.add_argument("--no-prefill", action="store_true", help="skip the router prefill records")
    ap.add_argument("--no-layers", action="store_true", help="skip the 48-layer decode-step records")
    ap.add_argument("--extra", action="store_true", help="also the seven-ratio batched sweep")
    ap.add_argument("--extra-ratios", type=str, default="",
                    help="comma-separated subset of the sweep's ratios (default: all seven)")
    ap.add_argument("--only-headline-kernel", action="store_true",
                    help="profiling aid: time only the headline workload")
    ap.add_argument("--kernel-launches", type=int, default=200, help="launches per per-kernel timing loop")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="profiling aid: after timing, copy this many MiB device-to-device once (a plain copy of "
                         "known size to scale HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class DecodeBench:
    """Device buffers, graphs and timings of one decode workload."""

    def __init__(self, case, budget, scoring, dev, replicas_gib=1.0):
        import torch
        from block_sparse_attention_chunk_amd import ops
        self.ops, self.torch, self.case, self.dev = ops, torch, case, dev
        self.scoring = scoring
        self.kind = ops.BSA_ENVELOPE if scoring == "envelope" else ops.BSA_CENTROID
        self.budget = budget
        base_k, base_v = ops.upload(case.k, dev), ops.upload(case.v, dev)
        self.q = ops.upload(case.q, dev)
        bt, sl = ops.upload(case.block_table, dev), ops.upload(case.seq_lens, dev)
        self.which = ops.BSA_META_ENVELOPE if self.kind == ops.BSA_ENVELOPE else ops.BSA_META_CENTROID
        kv_bytes = case.k.nbytes + case.v.nbytes
        self.replicas = max(1, math.ceil(replicas_gib * 2 ** 30 / kv_bytes))
        self.reps = []
        for r in range(self.replicas):
            k = base_k if r == 0 else base_k.clone()
            v = base_v if r == 0 else base_v.clone()
            kv = ops.KVCache(k, v, sl, case.page_size, bt)
            self.reps.append((kv, ops.build_chunk_meta(kv, which=self.which)))
        kv0 = self.reps[0][0]
        self.max_sel = budget.max_selected(kv0.max_pages)
        B, H = case.batch, case.num_kv_heads
        self.scores = torch.empty((B, H, kv0.max_pages), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, H, self.max_sel), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, case.num_q_heads, case.head_dim), dtype=torch.float32, device=dev)
        self.ws = torch.zeros((max(ops.decode_workspace_bytes(kv0, case.num_q_heads, self.max_sel), 1),),
                              dtype=torch.uint8, device=dev)
        self.splits = ops.decode_num_splits(kv0, case.num_q_heads, self.max_sel)
        # the dense baseline is timed at the automatic split count and at 2x and
        # 4x of it (up to 64), and the fastest counts
        auto = ops.decode_num_splits(kv0, case.num_q_heads, kv0.max_pages)
        self.dense_candidates = sorted({min(64, auto * f) for f in (1, 2, 4)})
        self.dense_splits = auto
        self.dws = torch.zeros((max(ops.decode_workspace_bytes(kv0, case.num_q_heads, kv0.max_pages,
                                                               self.dense_candidates[-1]), 1),),
                               dtype=torch.uint8, device=dev)

    # --- the hot path ---------------------------------------------------------------
    def score(self, r):
        kv, meta = self.reps[r]
        self.ops.score_chunks(self.q, kv, meta, self.kind, out=self.scores)

    def select(self, r):
        ops = self.ops
        kv, meta = self.reps[r]
        ops.score_chunks(self.q, kv, meta, self.kind, out=self.scores)
        ops.select_topk(self.scores, kv, self.budget, max_sel=self.max_sel, sel_idx=self.sel, sel_count=self.cnt)

    def attend(self, r):
        kv, _ = self.reps[r]
        self.ops.sparse_attn_decode(self.q, kv, self.sel, self.cnt, out=self.out, workspace=self.ws)

    def decode_kernel(self, r):
        kv, _ = self.reps[r]
        self.ops.sparse_attn_decode(self.q, kv, self.sel, self.cnt, out=self.partials_or_out(), workspace=self.ws)

    def merge(self, r):
        self.ops.decode_merge(self.ws, self.case.batch, self.case.num_q_heads, self.case.head_dim, self.splits,
                              out=self.out)

    def fused(self, r):
        kv, _ = self.reps[r]
        self.ops.select_attn_decode(self.q, kv, self.scores, self.budget, out=self.out, workspace=self.ws)

    def fused_kernel(self, r):
        kv, _ = self.reps[r]
        self.ops.select_attn_decode(self.q, kv, self.scores, self.budget, out=self.partials_or_out(),
                                    workspace=self.ws)

    def partials_or_out(self):
        return self.ops.PARTIALS if self.splits > 1 else self.out

    def step(self, r):
        """The decode step: scores, then selection + attention + merge."""
        self.score(r)
        self.fused(r)

    def step_unfused(self, r):
        self.select(r)
        self.attend(r)

    def dense(self, r):
        kv, _ = self.reps[r]
        self.ops.sparse_attn_decode(self.q, kv, None, None, num_splits=self.dense_splits, out=self.out,
                                    workspace=self.dws)

    def time_dense(self, launches):
        """The dense baseline at its fastest split count among the candidates."""
        best = None
        for s in self.dense_candidates:
            self.dense_splits = s
            t = self.time_kernel(self.dense, launches)
            if best is None or t < best[0]:
                best = (t, s)
        self.dense_splits = best[1]
        return best[0]

    def meta(self, r):
        kv, meta = self.reps[r]
        self.ops.build_chunk_meta(kv, which=self.which, meta=meta)

    # --- graphs and timing ----------------------------------------------------------
    def graph(self, fn, reps):
        torch = self.torch
        for r in reps:   # code objects are loaded before capture
            fn(r)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in reps:
                fn(r)
        torch.cuda.synchronize()
        return g

    def time_steps(self, steps, warmup, fn=None):
        """Exactly `steps` decode steps, rotating replicas, from HIP graphs.  A
        graph holds whole rounds over the replicas, at least 16 steps, so the
        replay's host overhead stays hidden behind the device work."""
        torch = self.torch
        fn = fn or self.step
        R = self.replicas
        rounds = max(1, math.ceil(16 / R))
        g_block = self.graph(fn, list(range(R)) * rounds)
        g_one = [self.graph(fn, [r]) for r in range(R)]
        per_block = R * rounds

        def run(n):
            full, rem = divmod(n, per_block)
            for _ in range(full):
                g_block.replay()
            for r in range(rem):
                g_one[r % R].replay()

        run(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(steps)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def time_kernel(self, fn, min_launches=200):
        """Average duration of one launch of fn: back-to-back launches over the
        replicas (at least 32 per graph), bracketed by HIP events on the launch
        stream."""
        torch = self.torch
        R = self.replicas
        reps = list(range(R)) * max(1, math.ceil(32 / R))
        per = max(1, math.ceil(min_launches / len(reps)))
        g = self.graph(fn, reps)
        stream = torch.cuda.current_stream(self.dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()
        e0.record(stream)
        for _ in range(per):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (per * len(reps))

    def bytes(self):
        """Algorithmic bytes of one step: metadata read + selected K/V + q in + out."""
        case = self.case
        D, H, Hq, B, P = case.head_dim, case.num_kv_heads, case.num_q_heads, case.batch, case.page_size
        n = case.n_chunks()
        meta_per_chunk = 2 * D * 2 if self.scoring == "envelope" else D * 4
        meta = int(n.sum()) * H * meta_per_chunk
        sel_tokens = 0
        for b in range(B):
            L = int(case.seq_lens[b])
            K = self.budget.max_selected(int(n[b]))      # pages kept per head
            full = min(K, int(n[b]))
            tokens = full * P if full < int(n[b]) else L  # all pages: the partial last page counts its tokens
            sel_tokens += min(tokens, L)
        kvb = sel_tokens * H * D * 2 * 2
        dense_kv = int(case.seq_lens.sum()) * H * D * 2 * 2
        qo = B * Hq * D * (2 + 4)
        return meta, kvb, qo, dense_kv

    def measure(self, steps, warmup, launches=200):
        t_step = self.time_steps(steps, warmup)
        t_step_unfused = self.time_steps(steps, warmup, self.step_unfused)
        self.step_unfused(0)
        self.torch.cuda.synchronize()
        m = {"t_step": t_step, "t_step_unfused": t_step_unfused,
             "t_fused": self.time_kernel(self.fused, launches),
             "t_fused_kernel": self.time_kernel(self.fused_kernel, launches),
             "t_attn": self.time_kernel(self.attend, launches),
             "t_decode_kernel": self.time_kernel(self.decode_kernel, launches),
             "t_dense": self.time_dense(launches),
             "t_score": self.time_kernel(self.score, launches),
             "t_select": self.time_kernel(self.select, launches),
             "t_meta": self.time_kernel(self.meta, launches)}
        self.decode_kernel(0)
        m["t_merge"] = self.time_kernel(self.merge, launches) if self.splits > 1 else 0.0
        meta_b, kv_b, qo_b, dense_b = self.bytes()
        m.update({"meta_bytes": meta_b, "kv_bytes": kv_b, "qo_bytes": qo_b, "dense_kv_bytes": dense_b})
        return m


def record(name, bench, m):
    case = bench.case
    step_bytes = m["meta_bytes"] + m["kv_bytes"] + m["qo_bytes"]
    kvb = m["kv_bytes"]
    return {
        "workload": name,
        "batch": case.batch, "seq_len": int(case.seq_lens.max()), "q_heads": case.num_q_heads,
        "kv_heads": case.num_kv_heads, "head_dim": case.head_dim, "scoring": bench.scoring,
        "tokens_per_s": case.batch / m["t_step"],
        "us_per_step": m["t_step"] * 1e6,
        "unfused_us_per_step": m["t_step_unfused"] * 1e6,
        "effective_hbm_gbs": step_bytes / m["t_step"] / 1e9,
        "effective_hbm_frac": step_bytes / m["t_step"] / 1e9 / HBM_PEAK_GBS,
        "score_us": m["t_score"] * 1e6,
        "fused_select_attn_us": m["t_fused"] * 1e6,
        "fused_kernel_us": m["t_fused_kernel"] * 1e6,
        "fused_kernel_selected_kv_gbs": kvb / m["t_fused_kernel"] / 1e9,
        "sparse_attn_us": m["t_attn"] * 1e6,
        # selected K/V over the whole attention call (automatic schedule, merge included)
        "attn_selected_kv_gbs": kvb / m["t_attn"] / 1e9,
        "decode_kernel_us": m["t_decode_kernel"] * 1e6,
        "merge_kernel_us": m["t_merge"] * 1e6,
        "selected_kv_gbs": kvb / m["t_decode_kernel"] / 1e9,
        "selected_kv_frac": kvb / m["t_decode_kernel"] / 1e9 / HBM_PEAK_GBS,
        "score_select_us": m["t_select"] * 1e6,
        "meta_build_us": m["t_meta"] * 1e6,
        "dense_attn_us": m["t_dense"] * 1e6,
        "dense_kv_gbs": m["dense_kv_bytes"] / m["t_dense"] / 1e9,
        "speedup_attn_vs_dense": m["t_dense"] / m["t_attn"],
        "speedup_step_vs_dense": m["t_dense"] / m["t_step"],
        "splits": bench.splits,
        "dense_splits": bench.dense_splits,
        "cache_replicas": bench.replicas,
        "bytes_per_step": {"metadata": m["meta_bytes"], "selected_kv": kvb, "q_out": m["qo_bytes"]},
    }


class ChunkedDecodeBench(DecodeBench):
    """Decode over variable, document-aligned chunks (envelope scoring, token
    budget): chunk scores, the longest score-order prefix that fits the budget,
    then split-K attention over the kept chunks.  Two calls: the fused
    selection + attention entry point takes 16-token pages only."""

    def __init__(self, case, budget, dev, replicas_gib=1.0):
        import torch
        from block_sparse_attention_chunk_amd import ops
        self.ops, self.torch, self.case, self.dev = ops, torch, case, dev
        self.scoring, self.kind, self.budget = "envelope", ops.BSA_ENVELOPE, budget
        self.which = ops.BSA_META_ENVELOPE
        self.chunks = ops.Chunks(ops.upload(case.chunk_starts, dev), ops.upload(case.num_chunks, dev))
        base_k, base_v = ops.upload(case.k, dev), ops.upload(case.v, dev)
        self.q = ops.upload(case.q, dev)
        bt, sl = ops.upload(case.block_table, dev), ops.upload(case.seq_lens, dev)
        self.replicas = max(1, math.ceil(replicas_gib * 2 ** 30 / (case.k.nbytes + case.v.nbytes)))
        self.reps = []
        for r in range(self.replicas):
            k = base_k if r == 0 else base_k.clone()
            v = base_v if r == 0 else base_v.clone()
            kv = ops.KVCache(k, v, sl, case.page_size, bt)
            self.reps.append((kv, ops.build_chunk_meta(kv, self.chunks, which=self.which)))
        kv0 = self.reps[0][0]
        mc = self.chunks.max_chunks
        self.max_sel = budget.max_selected(mc)
        B, H = case.batch, case.num_kv_heads
        self.scores = torch.empty((B, H, mc), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, H, self.max_sel), dtype=torch.int32, device=dev)
        self.cnt = torch.empty((B, H), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, case.num_q_heads, case.head_dim), dtype=torch.float32, device=dev)
        self.ws = torch.zeros((max(ops.decode_workspace_bytes(kv0, case.num_q_heads, self.max_sel), 1),),
                              dtype=torch.uint8, device=dev)
        self.dws = torch.zeros((max(ops.decode_workspace_bytes(kv0, case.num_q_heads, mc), 1),),
                               dtype=torch.uint8, device=dev)
        self.splits = ops.decode_num_splits(kv0, case.num_q_heads, self.max_sel)

    def score(self, r):
        kv, meta = self.reps[r]
        self.ops.score_chunks(self.q, kv, meta, self.kind, chunks=self.chunks, out=self.scores)

    def select(self, r):
        kv, meta = self.reps[r]
        self.ops.score_chunks(self.q, kv, meta, self.kind, chunks=self.chunks, out=self.scores)
        self.ops.select_topk(self.scores, kv, self.budget, chunks=self.chunks, max_sel=self.max_sel,
                             sel_idx=self.sel, sel_count=self.cnt)

    def attend(self, r):
        kv, _ = self.reps[r]
        self.ops.sparse_attn_decode(self.q, kv, self.sel, self.cnt, chunks=self.chunks, out=self.out,
                                    workspace=self.ws)

    def dense(self, r):
        kv, _ = self.reps[r]
        self.ops.sparse_attn_decode(self.q, kv, None, None, chunks=self.chunks, out=self.out, workspace=self.dws)

    def step(self, r):
        self.select(r)
        self.attend(r)

    def measure(self, steps, warmup, launches=200):
        t_step = self.time_steps(steps, warmup)
        self.select(0)
        self.torch.cuda.synchronize()
        case, D, H = self.case, self.case.head_dim, self.case.num_kv_heads
        sel, cnt = self.sel.cpu().numpy(), self.cnt.cpu().numpy()
        kept = sum(int(case.chunk_len[b][sel[b, h, :cnt[b, h]]].sum())
                   for b in range(case.batch) for h in range(H))
        kv_b = kept * D * 2 * 2
        meta_b = int(case.num_chunks.sum()) * H * 2 * D * 2
        t_attn, t_dense = self.time_kernel(self.attend, launches), self.time_kernel(self.dense, launches)
        return {"workload": f"variable chunks (U[16,256] tokens, {int(case.num_chunks.max())} chunks), "
                            f"1 x {int(case.seq_lens.max())} tokens, envelope, token budget {self.budget.tokens}",
                "budget_tokens": self.budget.tokens, "attended_tokens_per_head": kept / (case.batch * H),
                "tokens_per_s": case.batch / t_step, "us_per_step": t_step * 1e6,
                "score_select_us": self.time_kernel(self.select, launches) * 1e6,
                "sparse_attn_us": t_attn * 1e6, "dense_attn_us": t_dense * 1e6,
                "selected_kv_gbs": kv_b / t_attn / 1e9,
                "effective_hbm_gbs": (meta_b + kv_b) / t_step / 1e9,
                "speedup_attn_vs_dense": t_dense / t_attn, "speedup_step_vs_dense": t_dense / t_step}


class PrefillBench:
    """Router prefill over query tiles: block metadata, tile scores, the
    uncertainty router and the sparse / dense causal tile attention."""

    def __init__(self, pc, dev, kind, k=32, rho=2, quantile=0.25):
        import torch
        from block_sparse_attention_chunk_amd import ops
        self.ops, self.torch, self.pc, self.dev = ops, torch, pc, dev
        self.kind, self.k, self.rho, self.quantile = kind, k, rho, quantile
        self.kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(pc.v, dev),
                              torch.tensor([pc.T], dtype=torch.int32, device=dev), pc.block, token_major=True)
        self.q = ops.upload(pc.q, dev)
        which = ops.BSA_META_ENVELOPE if kind == ops.BSA_ENVELOPE else ops.BSA_META_CENTROID
        self.which = which
        self.meta = ops.build_chunk_meta(self.kv, which=which)
        nt = (pc.T + pc.tile - 1) // pc.tile
        self.n_tiles = nt
        self.ts = torch.empty((nt, pc.num_kv_heads, self.kv.max_pages), dtype=torch.float32, device=dev)
        self.ws = torch.empty((max(ops.router_workspace_bytes(nt, pc.num_kv_heads, k, rho), 1),), dtype=torch.uint8,
                              device=dev)
        self.out = torch.empty((pc.T, pc.num_q_heads, pc.head_dim), dtype=torch.float32, device=dev)
        self.pws = torch.empty((ops.tile_prefill_workspace_bytes(self.kv, pc.T),), dtype=torch.uint8, device=dev)
        self.r = None

    def build_meta(self, _=0):
        self.ops.build_chunk_meta(self.kv, which=self.which, meta=self.meta)

    def score(self, _=0):
        self.ops.score_chunks(self.q, self.kv, self.meta, self.kind, rows_per_query=self.pc.tile, causal=True,
                              out=self.ts)

    def route(self, _=0):
        self.r = self.ops.select_topk_router(self.ts, k=self.k, rho=self.rho, quantile=self.quantile,
                                             workspace=self.ws)

    def attend(self, _=0):
        self.ops.sparse_attn_tile_prefill(self.q, self.kv, self.r["kv_idx"], out=self.out, workspace=self.pws)

    def dense(self, _=0):
        self.ops.sparse_attn_tile_prefill(self.q, self.kv, None, out=self.out, workspace=self.pws)

    def timed(self, fn, reps, repeats=5):
        """Median over `repeats` runs of the average time of `reps` back-to-back
        calls (HIP events on the current stream)."""
        torch = self.torch
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3 / reps)
        return sorted(times)[len(times) // 2]

    def measure(self, reps=5):
        t_meta = self.timed(self.build_meta, reps)
        t_score = self.timed(self.score, reps)
        t_route = self.timed(self.route, reps)
        t_attn = self.timed(self.attend, reps)
        t_dense = self.timed(self.dense, 1, repeats=3)
        pc = self.pc
        g = pc.num_q_heads // pc.num_kv_heads
        kv_idx = self.r["kv_idx"].cpu().numpy()
        n_sel = int((kv_idx >= 0).sum())                        # (tile, KV head, block) triples attended
        trig = int(self.r["triggered"].sum().item())
        R, Bk, D = pc.tile, pc.block, pc.head_dim
        attn_flops = 4.0 * R * Bk * D * g * n_sel               # QK^T + PV, full blocks
        nt = self.n_tiles
        vis_pairs = sum(min(t + 1, self.kv.max_pages) for t in range(nt)) * pc.num_kv_heads
        score_flops = 2.0 * R * g * (2 * D) * vis_pairs        # [q+|q-] x [kmax;kmin] per visible block
        dense_flops = 4.0 * R * Bk * D * g * vis_pairs
        t_sparse = t_score + t_route + t_attn
        peak = BF16_MFMA_PEAK_TFLOPS * 1e12
        return {
            "workload": f"router prefill, {pc.T} tokens, {pc.num_q_heads} q / {pc.num_kv_heads} KV heads, d {D}, "
                        f"bf16, 64-token blocks / 64-row tiles, k={self.k}, rho={self.rho}, quantile "
                        f"{self.quantile}, {'envelope' if self.kind == 0 else 'centroid'} scoring",
            "tokens_per_s": pc.T / t_sparse,
            "sparse_pipeline_ms": t_sparse * 1e3,
            "meta_build_ms": t_meta * 1e3, "tile_score_ms": t_score * 1e3, "router_ms": t_route * 1e3,
            "sparse_attn_ms": t_attn * 1e3, "dense_causal_attn_ms": t_dense * 1e3,
            "sparse_pipeline_vs_dense_attn": t_sparse / t_dense,
            "triggered_tiles": trig, "attended_blocks": n_sel,
            "attn_tflops": attn_flops / t_attn / 1e12, "attn_mfma_frac": attn_flops / t_attn / peak,
            "score_tflops": score_flops / t_score / 1e12, "score_mfma_frac": score_flops / t_score / peak,
            "dense_tflops": dense_flops / t_dense / 1e12, "dense_mfma_frac": dense_flops / t_dense / peak,
            "roofline": {"bound": "mfma", "kernel": "tile_prefill_kernel", "achieved": attn_flops / t_attn / 1e12,
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": attn_flops / t_attn / peak,
                         "traffic": None},
        }


class LayerStackBench:
    """A serving-shaped decode step: `layers` replay-shaped layers, each with
    its own K/V cache and metadata (device copies of one generated layer),
    every layer running scoring + fused selection / attention + merge; the
    whole step is one HIP graph."""

    def __init__(self, case, budget, scoring, dev, layers=48):
        import torch
        from block_sparse_attention_chunk_amd import ops
        self.ops, self.torch, self.case, self.dev, self.layers = ops, torch, case, dev, layers
        self.kind = ops.BSA_ENVELOPE if scoring == "envelope" else ops.BSA_CENTROID
        which = ops.BSA_META_ENVELOPE if self.kind == ops.BSA_ENVELOPE else ops.BSA_META_CENTROID
        self.budget = budget
        k0, v0 = ops.upload(case.k, dev), ops.upload(case.v, dev)
        bt, sl = ops.upload(case.block_table, dev), ops.upload(case.seq_lens, dev)
        self.q = ops.upload(case.q, dev)
        self.stack = []
        for i in range(layers):
            kv = ops.KVCache(k0 if i == 0 else k0.clone(), v0 if i == 0 else v0.clone(), sl, case.page_size, bt)
            self.stack.append((kv, ops.build_chunk_meta(kv, which=which)))
        kv0 = self.stack[0][0]
        B, H = case.batch, case.num_kv_heads
        self.scores = torch.empty((B, H, kv0.max_pages), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, case.num_q_heads, case.head_dim), dtype=torch.float32, device=dev)
        K = budget.max_selected(kv0.max_pages)
        self.ws = torch.zeros((max(ops.decode_workspace_bytes(kv0, case.num_q_heads, K), 1),), dtype=torch.uint8,
                              device=dev)
        self.dws = torch.zeros((max(ops.decode_workspace_bytes(kv0, case.num_q_heads, kv0.max_pages), 1),),
                               dtype=torch.uint8, device=dev)

    def step(self):
        ops = self.ops
        for kv, meta in self.stack:
            ops.score_chunks(self.q, kv, meta, self.kind, out=self.scores)
            ops.select_attn_decode(self.q, kv, self.scores, self.budget, out=self.out, workspace=self.ws)

    def dense_step(self):
        for kv, _ in self.stack:
            self.ops.sparse_attn_decode(self.q, kv, None, None, out=self.out, workspace=self.dws)

    def measure(self, steps=20):
        torch = self.torch
        res = {}
        for name, fn in (("sparse", self.step), ("dense", self.dense_step)):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            g.replay()
            torch.cuda.synchronize()
            n = steps if name == "sparse" else max(2, steps // 4)
            t0 = time.perf_counter()
            for _ in range(n):
                g.replay()
            torch.cuda.synchronize()
            res[name] = (time.perf_counter() - t0) / n
            del g
        case = self.case
        return {"workload": f"{self.layers}-layer decode step, replay-shaped layers (32 q / 4 KV heads, d 128, "
                            f"bf16), {case.batch} x {int(case.seq_lens.max())} tokens, top-256 pages per KV head",
                "layers": self.layers, "batch": case.batch,
                "tokens_per_s": case.batch / res["sparse"], "ms_per_token_step": res["sparse"] * 1e3,
                "us_per_layer": res["sparse"] / self.layers * 1e6,
                "dense_ms_per_token_step": res["dense"] * 1e3,
                "speedup_vs_dense_attention": res["dense"] / res["sparse"]}


PMC_SUMMARY = os.path.join(ROOT, "profiles", "select_decode_replay_b1_hbm_traffic.txt")
KERNEL_SOURCES = ["select_decode.hip", "decode_common.h", "radix_select.h", "select_rules.h", "bsa_internal.h"]


def kernel_source_hash():
    """sha1 over the sources of the headline fused kernel."""
    import hashlib
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "block_sparse_attention_chunk_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the headline fused kernel from the committed
    FETCH_SIZE / WRITE_SIZE summary, or None when that summary was taken on a
    different version of the kernel's sources."""
    try:
        fields = {}
        for line in open(PMC_SUMMARY):
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if kernel_source_hash() != fields.get("kernel_source_sha1"):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(case, k_pages, scoring, seconds):
    """The fp64 oracle on the host cores on the same inputs and stages (score +
    select + attention per step, metadata built once), run for ~`seconds`."""
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
            "sample": f"{steps} complete decode steps of the headline workload (score + select + attention over "
                      f"the same inputs; metadata built once) in {el:.1f} s, fp64, OpenMP {threads} threads"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "bsa runs on one GPU: --gpus must be 1 (there is no multi-GPU path)"}))
        sys.exit(2)
    import torch
    from block_sparse_attention_chunk_amd import ops, synth
    dev = torch.device("cuda:0")

    log("headline: replay-shaped decode layer")
    case = synth.replay_decode()
    k_pages = a.budget // case.page_size
    hb = DecodeBench(case, ops.Budget.topk(k_pages), a.scoring, dev, a.replicas_gib)
    m = hb.measure(a.steps, a.warmup, a.kernel_launches)
    head = record(f"replay-shaped decode, {case.num_q_heads} q / {case.num_kv_heads} KV heads, d 128, bf16, "
                  f"{int(case.seq_lens[0])} tokens, {a.scoring} scoring, top-{k_pages} of "
                  f"{int(case.n_chunks()[0])} 16-token pages (budget {k_pages * 16} tokens), 1 sequence", hb, m)
    res = {
        "metric": "sparse decode tokens/s + effective HBM GB/s (% of peak) at 32K ctx, budget 4096",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": m["t_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) keys/values, 24 planted needle pages, 4 outlier channels x8",
        "config": {"workload": head["workload"], "batch": 1, "seq_len": int(case.seq_lens[0]),
                   "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
                   "page_size": case.page_size, "budget_tokens": k_pages * 16, "scoring": a.scoring,
                   "splits": hb.splits, "cache_replicas": hb.replicas, "graph_replay": True},
        "effective_hbm_gbs": head["effective_hbm_gbs"],
        "effective_hbm_frac": head["effective_hbm_frac"],
        "roofline": {"bound": "hbm",
                     "kernel": "select_decode_kernel (bsa_select_attn_decode without the merge)",
                     "achieved": head["fused_kernel_selected_kv_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["fused_kernel_selected_kv_gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": m["kv_bytes"],
                     "launch_us": m["t_fused_kernel"] * 1e6},
        "headline": head,
    }
    del hb
    torch.cuda.empty_cache()

    if not a.no_batched and not a.only_headline_kernel:
        extra = []
        log("batched: replay-shaped layer, 16 sequences x 32768 tokens")
        c16 = synth.replay_decode(seq_len=32768, batch=16)
        b16 = DecodeBench(c16, ops.Budget.topk(256), "envelope", dev, a.replicas_gib)
        extra.append(record("replay-shaped decode, 16 x 32768 tokens, envelope, top-256 pages (4096 tokens)", b16,
                            b16.measure(max(50, a.steps // 4), 5)))
        del b16, c16
        torch.cuda.empty_cache()
        log("batched: 64 q / 8 KV heads, 16 x 32768 tokens, ratio 1/8")
        c3 = synth.batched_decode(cid=3, seq_lens=[32768] * 16)
        b3 = DecodeBench(c3, ops.Budget.ratio_budget(0.125, 1, 1), "centroid", dev, a.replicas_gib)
        extra.append(record("batched decode, 64 q / 8 KV heads, 16 x 32768 tokens, centroid, ratio 1/8 with "
                            "bos+eos (4096 tokens per sequence and head)", b3, b3.measure(max(50, a.steps // 4), 5)))
        del b3, c3
        torch.cuda.empty_cache()
        log("batched: 64 q / 8 KV heads, 16 x U[8K, 32K] tokens, ratio 1/2")
        cr = synth.batched_decode()
        br = DecodeBench(cr, ops.Budget.ratio_budget(0.5, 1, 1), "centroid", dev, a.replicas_gib)
        extra.append(record("batched decode, 64 q / 8 KV heads, 16 x U[8192, 32768] tokens (8,409-30,271), centroid, "
                            "ratio 1/2 with bos+eos; attention call on the balanced schedule", br,
                            br.measure(max(50, a.steps // 4), 5)))
        del br, cr
        torch.cuda.empty_cache()
        res["batched"] = extra
    if not a.no_prefill and not a.only_headline_kernel:
        log("router prefill: 131072 tokens")
        pc = synth.router_prefill()
        pb = PrefillBench(pc, dev, ops.BSA_ENVELOPE)
        res["prefill"] = pb.measure()
        del pb, pc
        torch.cuda.empty_cache()
        by_len = []
        for T in (32768, 65536):
            log(f"router prefill: {T} tokens")
            pc = synth.router_prefill(T=T, groups=max(4, T // 8192), tied_groups=tuple(range(3, max(4, T // 8192), 4)))
            pb = PrefillBench(pc, dev, ops.BSA_ENVELOPE)
            m = pb.measure()
            by_len.append({k: m[k] for k in ("workload", "tokens_per_s", "sparse_pipeline_ms", "tile_score_ms",
                                             "router_ms", "sparse_attn_ms", "dense_causal_attn_ms",
                                             "sparse_pipeline_vs_dense_attn", "triggered_tiles", "attn_mfma_frac")})
            del pb, pc
            torch.cuda.empty_cache()
        res["prefill_by_length"] = by_len
    if not a.no_layers and not a.only_headline_kernel:
        stacks = []
        for B, L in ((1, None), (16, 32768)):
            log(f"48-layer decode step, {B} sequence(s)")
            c = synth.replay_decode() if L is None else synth.replay_decode(seq_len=L, batch=B)
            lb = LayerStackBench(c, ops.Budget.topk(256), "envelope", dev)
            stacks.append(lb.measure())
            del lb, c
            torch.cuda.empty_cache()
        res["layer_stack"] = stacks
    if a.extra:
        keep = ("workload", "tokens_per_s", "us_per_step", "unfused_us_per_step", "sparse_attn_us", "attn_selected_kv_gbs",
                "selected_kv_gbs", "selected_kv_frac",
                "dense_attn_us", "speedup_attn_vs_dense", "speedup_step_vs_dense", "effective_hbm_gbs")
        log("budget sweep: replay-shaped layer, 1 x 29504 tokens")
        c1 = synth.replay_decode()
        sweep = []
        for scoring in ("envelope", "centroid"):
            for k in (256, 512):
                b1 = DecodeBench(c1, ops.Budget.topk(k), scoring, dev, a.replicas_gib)
                rec = record(f"replay-shaped decode, 1 x 29504 tokens, {scoring}, top-{k} pages ({16 * k} tokens)",
                             b1, b1.measure(100, 10))
                sweep.append({k_: rec[k_] for k_ in keep})
                del b1
                torch.cuda.empty_cache()
        del c1
        res["budget_sweep"] = sweep
        log("token-budget sweep: variable chunks, 1 x 29504 tokens")
        c2 = synth.varchunk_decode()
        tsa = []
        for tokens in (4096, 8192, 16384):
            b2 = ChunkedDecodeBench(c2, ops.Budget.token_budget(tokens), dev, a.replicas_gib)
            tsa.append(b2.measure(100, 10))
            del b2
            torch.cuda.empty_cache()
        del c2
        res["chunk_budget_sweep"] = tsa
        log("ratio sweep: 16 sequences of 8K-32K tokens, 64 q / 8 KV heads")
        c3 = synth.batched_decode()
        sweep = []
        ratios = [float(x) for x in a.extra_ratios.split(",")] if a.extra_ratios else synth.RATIOS
        for scoring, bos in (("centroid", 1), ("envelope", 0)):
            for ratio in ratios:
                b3 = DecodeBench(c3, ops.Budget.ratio_budget(ratio, bos, 1), scoring, dev, a.replicas_gib)
                rec = record(f"batched decode, ratio {ratio}, {scoring}", b3, b3.measure(40, 5))
                sweep.append({k: rec[k] for k in keep})
                del b3
                torch.cuda.empty_cache()
        res["ratio_sweep"] = sweep
    if a.calibration_copy_mib:
        n = a.calibration_copy_mib * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n} bytes done")
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(case, k_pages, a.scoring, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
