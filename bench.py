#!/usr/bin/env python3
"""Benchmark: sparse decode tokens/s and effective HBM bandwidth on one MI355X.

Headline workload (the metric's own point, 32K context, budget 4096): one
decode layer shaped like the replay study's model (32 q / 4 KV heads,
head_dim 128, bf16, 16-token pages) at 32,768 cached tokens, top 256 of 2,048
pages per KV head (4,096 tokens), envelope scoring, one sequence.  One step =
chunk scoring + per-KV-head top-k + split-K sparse attention + split merge,
run as the library's decode step, bsa_decode_step (three launches: scoring,
the fused selection + attention, the split merge).  The unfused sequence
(bsa_score_chunks, bsa_select_topk, bsa_sparse_attn_decode) is timed beside
it.  Chunk metadata is built once
before timing (in a live loop a page's metadata is written once per 16 decode
steps) and its build time is reported apart.

Cold cache: every workload rotates over replicas of its K/V cache and
metadata, as many as make the bytes one rotation touches (metadata + selected
K/V + scores + q / out, per step) reach 1 GiB, so the 256 MB last-level cache
cannot serve a step from an earlier one; step and per-kernel timings use the
same rotation, and every record names touched_bytes and cache_replicas.
Inputs are synthetic and seeded (block_sparse_attention_chunk_amd/synth.py)
and resident in HBM before the timed region.  Steps are captured in HIP graphs
and replayed, so host dispatch is not in the measurement: exactly --steps
steps are timed as one graph replay (the headline value), and separately 100
replays of 16-step graphs (rotating over the replicas) are each timed with HIP
events for the median and p10 / p90 of the per-step time.  Per-kernel figures come from HIP events around graph replays of that
launch alone on its stream.

Records in the same JSON line: the same layer with 16 sequences at 32,768
tokens; a 64 q / 8 KV-head batch of 16 x 32,768 tokens at ratio 1/8 (4096
tokens per sequence and head); the ragged 16 x U[8K, 32K] batch at ratio 1/2;
the speedup over this build's dense kernel at every budget (top-256 / top-512
pages on the 29,504-token layer with both scorings, token budgets 4096 / 8192
/ 16384 over variable chunks, and the seven ratios of the ragged batch with
both scorings); the 131,072-token router prefill (28 q / 4 KV heads, k = 32,
rho = 2) with its MFMA utilisation, and the same router at 32,768 and 65,536
tokens; a 48-layer decode step at 1 and 16 sequences; and the fp64 oracle
timed on the host cores (all threads and one thread; decode steps of the
headline workload, and the router-prefill stages on a stated subset).

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
    ap.add_argument("--seq-len", type=int, default=32768, help="cached tokens of the headline sequence")
    ap.add_argument("--replicas-gib", type=float, default=1.0,
                    help="bytes touched per rotation over the cache replicas (cold-cache mode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="oracle decode steps on all host threads")
    ap.add_argument("--cpu-seconds-1t", type=float, default=5.0, help="oracle decode steps on one thread")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched records")
    ap.add_argument("--no-sweep", action="store_true", help="skip the every-budget speedup records")
    ap.add_argument("--no-prefill", action="store_true", help="skip the router prefill records")
    ap.add_argument("--no-layers", action="store_true", help="skip the 48-layer decode-step records")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the gather-ceiling measurement beside the decode records")
    ap.add_argument("--sweep-ratios", type=str, default="",
                    help="comma-separated subset of the ragged batch's ratios (default: all seven)")
    ap.add_argument("--only", choices=["headline", "h1b16", "h2", "ragged"], default=None,
                    help="profiling aid: run only this decode workload's timing loops and print its record")
    ap.add_argument("--kernel-launches", type=int, default=200, help="launches per per-kernel timing loop")
    ap.add_argument("--samples", type=int, default=100, help="16-step replays timed for the step percentiles")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="profiling aid: after timing, copy this many MiB device-to-device once (a plain copy of "
                         "known size to scale HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def replicas_for(touched_bytes, gib):
    """Cache replicas whose rotation touches at least `gib` GiB."""
    return max(1, math.ceil(gib * 2 ** 30 / max(1, touched_bytes)))


def percentiles(samples):
    x = np.sort(np.asarray(samples))
    return {"median": float(np.median(x)), "p10": float(np.percentile(x, 10)), "p90": float(np.percentile(x, 90)),
            "n": int(x.size)}


class Rotation:
    """HIP graphs of a workload's step (or kernel) over its cache replicas, and
    the timing protocols used on them."""

    def __init__(self, torch, dev, replicas):
        self.torch, self.dev, self.R = torch, dev, replicas

    def graph(self, fn, reps):
        torch = self.torch
        for r in sorted(set(reps)):   # code objects are loaded before capture
            fn(r)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in reps:
                fn(r)
        torch.cuda.synchronize()
        return g

    def time_steps(self, fn, steps, warmup):
        """Exactly `steps` calls of fn, rotating replicas, timed as one replay
        of a graph that holds all of them (after a graph of `warmup` calls on
        the replicas before them), so no host dispatch falls between steps;
        mean time per call."""
        torch, R = self.torch, self.R
        g_warm = self.graph(fn, [r % R for r in range(warmup)]) if warmup else None
        g_steps = self.graph(fn, [(warmup + i) % R for i in range(steps)])
        if g_warm is not None:
            g_warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_steps.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def sample_steps(self, fn, n, block=16):
        """At least n per-call samples: graphs of `block` consecutive calls
        covering the replicas in rotation are replayed in turn, each replay
        bracketed by HIP events on the launch stream; a sample is the mean
        call time of one replay (single-call replays would measure the host's
        graph launch, not the device, for calls of a few microseconds)."""
        torch, R = self.torch, self.R
        n_graphs = max(1, math.ceil(R / block))
        graphs = [self.graph(fn, [(block * j + i) % R for i in range(block)]) for j in range(n_graphs)]
        stream = torch.cuda.current_stream(self.dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for g in graphs:
            g.replay()
        for i in range(n):
            ev[i][0].record(stream)
            graphs[i % n_graphs].replay()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e-3 / block for a, b in ev]

    def time_kernel(self, fn, min_launches=200):
        """Average duration of one launch of fn: back-to-back launches over the
        replicas (at least 32 per graph), bracketed by HIP events on the launch
        stream."""
        torch, R = self.torch, self.R
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


class GatherCeiling:
    """The bandwidth ceiling of the decode's read pattern: the bare gather
    kernel of libbsa_ceiling.so reads distinct random 4 KiB runs (the size of
    one K or V run of a (page, KV head)) from a 4 GiB buffer, as many bytes per
    launch as a decode launch reads, with a fresh run list per launch (lists
    rotate like cache replicas, >= 1 GiB per rotation).  Best of three wave
    counts (256, 512, 1,024 workgroups of 4 waves), each timed like a kernel."""

    BUF_BYTES = 4 << 30
    RUN = 4096

    def __init__(self, torch, dev, gib=1.0):
        import ctypes
        path = os.path.join(ROOT, "block_sparse_attention_chunk_amd", "libbsa_ceiling.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run python -m block_sparse_attention_chunk_amd.build")
        self.lib = ctypes.CDLL(path)
        f = self.lib.bsa_ceiling_gather
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                      ctypes.c_void_p]
        f.restype = ctypes.c_int
        self.torch, self.dev, self.gib = torch, dev, gib
        self.buf = torch.empty(self.BUF_BYTES, dtype=torch.uint8, device=dev)
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        self.cache = {}

    def measure(self, nbytes):
        torch = self.torch
        n_runs = max(1, int(round(nbytes / self.RUN)))
        if n_runs in self.cache:
            return self.cache[n_runs]
        R = replicas_for(n_runs * self.RUN, self.gib)
        total = self.BUF_BYTES // self.RUN
        g = torch.Generator(device=self.dev)
        g.manual_seed(1000 + n_runs)
        runs = torch.stack([torch.randperm(total, generator=g, device=self.dev)[:n_runs] for _ in range(R)])
        runs = runs.to(torch.int32).contiguous()
        assert int(runs.min()) >= 0 and int(runs.max()) < total   # every run inside the buffer
        rot = Rotation(torch, self.dev, R)
        best = None
        for wgs in (256, 512, 1024):
            per_wave = max(1, math.ceil(n_runs / (4 * wgs)))

            def fn(r, per_wave=per_wave):
                stream = torch.cuda.current_stream(self.dev).cuda_stream
                rc = self.lib.bsa_ceiling_gather(self.buf.data_ptr(), runs[r].data_ptr(), n_runs, per_wave,
                                                 self.sink.data_ptr(), stream)
                if rc:
                    raise RuntimeError(f"bsa_ceiling_gather failed: hip error {rc}")

            t = rot.time_kernel(fn)
            if best is None or t < best[0]:
                best = (t, wgs)
        res = {"bytes": n_runs * self.RUN, "us": best[0] * 1e6, "gbs": n_runs * self.RUN / best[0] / 1e9,
               "workgroups": best[1], "run_lists": R}
        self.cache[n_runs] = res
        return res


def attach_ceiling(rec, ceil, kv_bytes):
    """The gather ceiling for the selected K/V bytes of one decode launch, and
    the decode kernels' read rates as fractions of it."""
    c = ceil.measure(kv_bytes)
    rec["gather_ceiling"] = c
    rec["selected_kv_of_ceiling"] = rec["selected_kv_gbs"] / c["gbs"]
    if "fused_kernel_selected_kv_gbs" in rec:
        rec["fused_kernel_of_ceiling"] = rec["fused_kernel_selected_kv_gbs"] / c["gbs"]
    rec["attn_call_of_ceiling"] = rec["attn_selected_kv_gbs"] / c["gbs"]
    return rec


class DecodeBench:
    """Device buffers, graphs and timings of one decode workload on 16-token
    pages, rotating over cold cache replicas."""

    def __init__(self, case, budget, scoring, dev, replicas_gib=1.0):
        import torch
        from block_sparse_attention_chunk_amd import ops
        self.ops, self.torch, self.case, self.dev = ops, torch, case, dev
        self.scoring = scoring
        self.kind = ops.BSA_ENVELOPE if scoring == "envelope" else ops.BSA_CENTROID
        self.budget = budget
        self.which = ops.BSA_META_ENVELOPE if self.kind == ops.BSA_ENVELOPE else ops.BSA_META_CENTROID
        B, H = case.batch, case.num_kv_heads
        max_pages = int(case.block_table.shape[1])
        meta_b, kv_b, qo_b, _ = self.bytes()
        self.touched = meta_b + kv_b + qo_b + B * H * max_pages * 4   # + the score row written and read
        self.replicas = replicas_for(self.touched, replicas_gib)
        self.rot = Rotation(torch, dev, self.replicas)
        base_k, base_v = ops.upload(case.k, dev), ops.upload(case.v, dev)
        self.q = ops.upload(case.q, dev)
        bt, sl = ops.upload(case.block_table, dev), ops.upload(case.seq_lens, dev)
        self.reps = []
        for r in range(self.replicas):
            k = base_k if r == 0 else base_k.clone()
            v = base_v if r == 0 else base_v.clone()
            kv = ops.KVCache(k, v, sl, case.page_size, bt)
            self.reps.append((kv, ops.build_chunk_meta(kv, which=self.which)))
        kv0 = self.reps[0][0]
        self.max_sel = budget.max_selected(kv0.max_pages)
        self.scores = torch.empty((B, H, kv0.max_pages), dtype=torch.float32, device=dev)
        self.sel = torch.full((B, H, self.max_sel), -1, dtype=torch.int32, device=dev)
        self.cnt = torch.zeros((B, H), dtype=torch.int32, device=dev)
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
        self.sws = torch.empty((ops.decode_step_workspace_bytes(kv0, case.num_q_heads, budget),), dtype=torch.uint8,
                               device=dev)

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
        """The decode step, bsa_decode_step: scoring, then the fused selection
        + attention, then the split merge."""
        kv, meta = self.reps[r]
        self.ops.decode_step(self.q, kv, meta, self.kind, self.budget, out=self.out, workspace=self.sws)

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
            t = self.rot.time_kernel(self.dense, launches)
            if best is None or t < best[0]:
                best = (t, s)
        self.dense_splits = best[1]
        return best[0]

    def meta(self, r):
        kv, meta = self.reps[r]
        self.ops.build_chunk_meta(kv, which=self.which, meta=meta)

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

    def measure(self, steps, warmup, launches=200, samples=100):
        rot = self.rot
        t_step = rot.time_steps(self.step, steps, warmup)
        pct = percentiles(rot.sample_steps(self.step, samples))
        t_step_unfused = rot.time_steps(self.step_unfused, steps, warmup)
        self.step_unfused(0)
        self.torch.cuda.synchronize()
        m = {"t_step": t_step, "step_pct": pct, "t_step_unfused": t_step_unfused,
             "t_fused": rot.time_kernel(self.fused, launches),
             "t_fused_kernel": rot.time_kernel(self.fused_kernel, launches),
             "t_attn": rot.time_kernel(self.attend, launches),
             "t_decode_kernel": rot.time_kernel(self.decode_kernel, launches),
             "t_dense": self.time_dense(launches),
             "t_score": rot.time_kernel(self.score, launches),
             "t_select": rot.time_kernel(self.select, launches),
             "t_meta": rot.time_kernel(self.meta, launches)}
        self.decode_kernel(0)
        m["t_merge"] = rot.time_kernel(self.merge, launches) if self.splits > 1 else 0.0
        meta_b, kv_b, qo_b, dense_b = self.bytes()
        m.update({"meta_bytes": meta_b, "kv_bytes": kv_b, "qo_bytes": qo_b, "dense_kv_bytes": dense_b})
        return m

    def measure_light(self, steps, warmup, launches=64, t_dense=None):
        """Step, attention call and dense attention only (the budget sweep)."""
        rot = self.rot
        t_step = rot.time_steps(self.step, steps, warmup)
        self.select(0)          # the attention calls below read this selection
        self.torch.cuda.synchronize()
        m = {"t_step": t_step,
             "t_attn": rot.time_kernel(self.attend, launches),
             "t_decode_kernel": rot.time_kernel(self.decode_kernel, launches),
             "t_dense": t_dense if t_dense is not None else self.time_dense(launches)}
        meta_b, kv_b, qo_b, dense_b = self.bytes()
        m.update({"meta_bytes": meta_b, "kv_bytes": kv_b, "qo_bytes": qo_b, "dense_kv_bytes": dense_b})
        return m


def record(name, bench, m):
    case = bench.case
    step_bytes = m["meta_bytes"] + m["kv_bytes"] + m["qo_bytes"]
    kvb = m["kv_bytes"]
    pct = m["step_pct"]
    return {
        "workload": name,
        "batch": case.batch, "seq_len": int(case.seq_lens.max()), "q_heads": case.num_q_heads,
        "kv_heads": case.num_kv_heads, "head_dim": case.head_dim, "scoring": bench.scoring,
        "tokens_per_s": case.batch / m["t_step"],
        "us_per_step": m["t_step"] * 1e6,
        "us_per_step_median": pct["median"] * 1e6, "us_per_step_p10": pct["p10"] * 1e6,
        "us_per_step_p90": pct["p90"] * 1e6, "step_samples": pct["n"], "steps_per_sample": 16,
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
        "step_over_dense": m["t_step"] / m["t_dense"],
        "splits": bench.splits,
        "dense_splits": bench.dense_splits,
        "cache_replicas": bench.replicas,
        "touched_bytes": bench.touched,
        "bytes_per_step": {"metadata": m["meta_bytes"], "selected_kv": kvb, "q_out": m["qo_bytes"]},
    }


def record_light(name, bench, m, budget):
    kvb = m["kv_bytes"]
    return {"workload": name, "budget": budget, "us_per_step": m["t_step"] * 1e6,
            "tokens_per_s": bench.case.batch / m["t_step"], "sparse_attn_us": m["t_attn"] * 1e6,
            "decode_kernel_us": m["t_decode_kernel"] * 1e6, "dense_attn_us": m["t_dense"] * 1e6,
            "speedup_attn_vs_dense": m["t_dense"] / m["t_attn"], "speedup_step_vs_dense": m["t_dense"] / m["t_step"],
            "attn_selected_kv_gbs": kvb / m["t_attn"] / 1e9, "selected_kv_gbs": kvb / m["t_decode_kernel"] / 1e9,
            "selected_kv_frac": kvb / m["t_decode_kernel"] / 1e9 / HBM_PEAK_GBS,
            "cache_replicas": bench.replicas, "touched_bytes": bench.touched}


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
        B, H, D = case.batch, case.num_kv_heads, case.head_dim
        mc = self.chunks.max_chunks
        # touched per step: metadata, at most the budget of K/V per head, scores, q / out
        self.touched = (int(case.num_chunks.sum()) * H * 2 * D * 2 + B * H * min(budget.tokens, int(case.seq_lens.max()))
                        * D * 2 * 2 + B * H * mc * 4 + B * case.num_q_heads * D * 6)
        self.replicas = replicas_for(self.touched, replicas_gib)
        self.rot = Rotation(torch, dev, self.replicas)
        base_k, base_v = ops.upload(case.k, dev), ops.upload(case.v, dev)
        self.q = ops.upload(case.q, dev)
        bt, sl = ops.upload(case.block_table, dev), ops.upload(case.seq_lens, dev)
        self.reps = []
        for r in range(self.replicas):
            k = base_k if r == 0 else base_k.clone()
            v = base_v if r == 0 else base_v.clone()
            kv = ops.KVCache(k, v, sl, case.page_size, bt)
            self.reps.append((kv, ops.build_chunk_meta(kv, self.chunks, which=self.which)))
        kv0 = self.reps[0][0]
        self.max_sel = budget.max_selected(mc)
        self.scores = torch.empty((B, H, mc), dtype=torch.float32, device=dev)
        self.sel = torch.full((B, H, self.max_sel), -1, dtype=torch.int32, device=dev)
        self.cnt = torch.zeros((B, H), dtype=torch.int32, device=dev)
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

    def measure(self, steps, warmup, launches=64):
        rot = self.rot
        t_step = rot.time_steps(self.step, steps, warmup)
        self.select(0)
        self.torch.cuda.synchronize()
        case, D, H = self.case, self.case.head_dim, self.case.num_kv_heads
        sel, cnt = self.sel.cpu().numpy(), self.cnt.cpu().numpy()
        kept = sum(int(case.chunk_len[b][sel[b, h, :cnt[b, h]]].sum())
                   for b in range(case.batch) for h in range(H))
        kv_b = kept * D * 2 * 2
        meta_b = int(case.num_chunks.sum()) * H * 2 * D * 2
        t_attn, t_dense = rot.time_kernel(self.attend, launches), rot.time_kernel(self.dense, launches)
        return {"workload": f"variable chunks (U[16,256] tokens, {int(case.num_chunks.max())} chunks), "
                            f"1 x {int(case.seq_lens.max())} tokens, envelope, token budget {self.budget.tokens}",
                "budget": f"{self.budget.tokens} tokens", "attended_tokens_per_head": kept / (case.batch * H),
                "tokens_per_s": case.batch / t_step, "us_per_step": t_step * 1e6,
                "score_select_us": rot.time_kernel(self.select, launches) * 1e6,
                "sparse_attn_us": t_attn * 1e6, "dense_attn_us": t_dense * 1e6,
                "attn_selected_kv_gbs": kv_b / t_attn / 1e9,
                "effective_hbm_gbs": (meta_b + kv_b) / t_step / 1e9,
                "speedup_attn_vs_dense": t_dense / t_attn, "speedup_step_vs_dense": t_dense / t_step,
                "cache_replicas": self.replicas, "touched_bytes": self.touched}


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


def torch_sdpa_causal(pc, dev, ours_dense_ms, repeats=3):
    """An outside reference for the dense causal tile attention: torch's own
    fused attention (scaled_dot_product_attention restricted to its flash
    backend, causal, bf16 in and out, scale 1/sqrt(d)) on the same q / K / V,
    K and V repeated over each KV head's query heads.  Timed with HIP events
    (median of `repeats` after one warm-up call).  A backend that refuses the
    shape leaves an explanation instead of a time."""
    import torch
    import torch.nn.functional as F
    from block_sparse_attention_chunk_amd import ops
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
    except ImportError as e:
        return {"available": False, "why": f"torch.nn.attention: {e}"}
    g = pc.num_q_heads // pc.num_kv_heads
    q = ops.upload(pc.q, dev).transpose(0, 1).unsqueeze(0).contiguous()                     # [1][Hq][T][D]
    k = ops.upload(pc.k, dev).transpose(0, 1).repeat_interleave(g, dim=0).unsqueeze(0).contiguous()
    v = ops.upload(pc.v, dev).transpose(0, 1).repeat_interleave(g, dim=0).unsqueeze(0).contiguous()
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            F.scaled_dot_product_attention(q, k, v, is_causal=True)
            torch.cuda.synchronize()
            times = []
            for _ in range(repeats):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                F.scaled_dot_product_attention(q, k, v, is_causal=True)
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
    except RuntimeError as e:
        return {"available": False, "why": str(e).splitlines()[0][:200]}
    finally:
        del q, k, v
        torch.cuda.empty_cache()
    t_ms = sorted(times)[len(times) // 2]
    T, D = pc.T, pc.head_dim
    flops = 4.0 * D * pc.num_q_heads * (T * (T + 1) / 2)          # exact causal count, QK^T + PV
    return {"available": True, "what": "torch scaled_dot_product_attention, flash backend, causal, bf16",
            "ms": t_ms, "tflops_exact_causal": flops / (t_ms * 1e-3) / 1e12,
            "dense_tile_kernel_speedup": t_ms / ours_dense_ms}


class LayerStackBench:
    """A serving-shaped decode step: `layers` replay-shaped layers, each with
    its own K/V cache and metadata (device copies of one generated layer),
    every layer running bsa_decode_step; the whole step is one HIP graph."""

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
        self.ws = torch.empty((ops.decode_step_workspace_bytes(kv0, case.num_q_heads, budget),), dtype=torch.uint8,
                              device=dev)
        self.dws = torch.zeros((max(ops.decode_workspace_bytes(kv0, case.num_q_heads, kv0.max_pages), 1),),
                               dtype=torch.uint8, device=dev)

    def step(self):
        ops = self.ops
        for kv, meta in self.stack:
            ops.decode_step(self.q, kv, meta, self.kind, self.budget, out=self.out, workspace=self.ws)

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


PMC_SUMMARY = os.path.join(ROOT, "profiles", "select_decode_replay_32k_b1_hbm_traffic.txt")
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_decode_rate(oracle, case, oc, meta, kind, k_pages, seconds):
    n = case.n_chunks()
    steps, t0 = 0, time.perf_counter()
    while True:
        _, sc, _ = oracle.score_decode(case.q, oc, meta, kind)
        sel, cnt = oracle.select(np.nan_to_num(sc, nan=-np.inf), n, oracle.TOPK, top_k=k_pages, max_sel=k_pages)
        oracle.decode_attn(case.q, oc, sel, cnt)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return steps, el


def cpu_baseline(case, k_pages, scoring, seconds, seconds_1t, prefill_blocks=None):
    """The fp64 oracle on the host cores on the same inputs and stages as the
    headline step (score + select + attention per step, metadata built once),
    with every thread the process may use and with one thread; then the
    router-prefill stages on a stated subset, extrapolated to the full
    131,072-token prefill."""
    import oracle
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    oracle.set_threads(threads)
    used = oracle.max_threads()
    oc = oracle.PagedCache(case.k, case.v, case.block_table, case.seq_lens, case.page_size, case.num_kv_heads,
                           case.head_dim)
    meta = oracle.chunk_meta(oc)
    kind = oracle.ENVELOPE if scoring == "envelope" else oracle.CENTROID
    steps, el = _oracle_decode_rate(oracle, case, oc, meta, kind, k_pages, seconds)
    oracle.set_threads(1)
    steps1, el1 = _oracle_decode_rate(oracle, case, oc, meta, kind, k_pages, seconds_1t)
    oracle.set_threads(used)
    res = {"value": case.batch * steps / el, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{steps} complete decode steps of the headline workload ({int(case.seq_lens[0])} tokens, "
                     f"top-{k_pages} pages; score + select + attention over the same inputs, metadata built once) "
                     f"in {el:.1f} s, fp64, OpenMP {used} threads",
           "single_thread": {"value": case.batch * steps1 / el1, "unit": "tokens/s", "cores": 1,
                             "sample": f"{steps1} decode steps in {el1:.1f} s, one thread"}}
    if prefill_blocks is not None:
        res["prefill"] = cpu_prefill_stages(oracle, used, prefill_blocks)
    return res


def cpu_prefill_stages(oracle, threads, attended_blocks):
    """Router-prefill stages of the oracle on a subset of the 131,072-token
    workload: tile scores of 6 tiles spread over the sequence (cost per tile
    grows with its visible blocks, t + 1), the router at full size (2,048
    tiles x 4 heads x 2,048 blocks of seeded scores), and the tile attention
    of 16 rows over 32 blocks each; each extrapolated by its work unit to the
    full prefill (attention: the GPU run's attended (tile, KV head, block)
    count)."""
    from block_sparse_attention_chunk_amd import synth
    pc = synth.router_prefill()
    T, Hq, H, D = pc.T, pc.num_q_heads, pc.num_kv_heads, pc.head_dim
    nt = T // 64
    g = Hq // H
    c = oracle.PagedCache(pc.k, pc.v, None, [T], 64, H, D, strides=(64 * H * D, D, H * D), max_pages=nt)
    t0 = time.perf_counter()
    meta = oracle.chunk_meta(c)
    t_meta = time.perf_counter() - t0
    tiles = np.array([100, 500, 900, 1300, 1700, 2047])
    t0 = time.perf_counter()
    oracle.tile_scores(pc.q, meta, oracle.ENVELOPE, num_kv_heads=H, tile_rows=64, block_size=64, tiles=tiles)
    t_ts = time.perf_counter() - t0
    vis_sub = float(np.sum(tiles + 1))
    vis_all = float(nt * (nt + 1) / 2)
    rng = np.random.default_rng(4)
    ts = rng.standard_normal((nt, H, nt))
    t0 = time.perf_counter()
    oracle.router(ts, np.arange(nt) + 1, 32, 2)
    t_router = time.perf_counter() - t0
    rows = np.array([64 * t + 17 for t in (40, 300, 700, 1100, 1500, 1900, 2047)] +
                    [64 * t + 63 for t in (60, 400, 800, 1200, 1600, 2000, 2046, 2047, 1000)])
    kv_idx = np.full((nt, H, 64), -1, np.int32)
    for t in np.unique(rows // 64):
        kv_idx[t, :, :32] = np.sort(rng.choice(t + 1, size=32, replace=False))[None, :]
    t0 = time.perf_counter()
    oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=H, block_size=64, tile_rows=64, kv_idx=kv_idx, rows=rows)
    t_attn = time.perf_counter() - t0
    # attention work unit: (row, q head, block); the sample does rows x Hq x 32
    per_unit = t_attn / (len(rows) * Hq * 32)
    full_units = attended_blocks * 64 * g                       # rows per tile x q heads per KV head
    ext = {"tile_scores_s": t_ts * vis_all / vis_sub, "router_s": t_router, "tile_attn_s": per_unit * full_units,
           "meta_s": t_meta}
    total = ext["tile_scores_s"] + ext["router_s"] + ext["tile_attn_s"]
    return {"value": T / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"tile scores of tiles {tiles.tolist()} ({t_ts:.2f} s, x {vis_all / vis_sub:.0f} by visible "
                      f"blocks), the router over 2048 x 4 x 2048 seeded scores ({t_router:.2f} s), tile attention "
                      f"of {len(rows)} rows over 32 blocks ({t_attn:.2f} s, extrapolated per (row, q head, block) to "
                      f"{attended_blocks} attended (tile, KV head, block) triples), metadata ({t_meta:.2f} s, not in "
                      f"the total); OpenMP {threads} threads",
            "extrapolated_s": ext, "total_s": total}


def decode_workloads(seq_len, budget_tokens, scoring):
    """(key, label, case, budget, scoring) of the decode records."""
    from block_sparse_attention_chunk_amd import ops, synth
    k_pages = budget_tokens // 16
    yield ("headline", f"replay-shaped decode, 32 q / 4 KV heads, d 128, bf16, {seq_len} tokens, {scoring} scoring, "
                       f"top-{k_pages} of {(seq_len + 15) // 16} 16-token pages (budget {k_pages * 16} tokens), "
                       f"1 sequence", lambda: synth.replay_decode(seq_len=seq_len), ops.Budget.topk(k_pages), scoring)
    yield ("h1b16", "replay-shaped decode, 16 x 32768 tokens, envelope, top-256 pages (4096 tokens)",
           lambda: synth.replay_decode(seq_len=32768, batch=16), ops.Budget.topk(256), "envelope")
    yield ("h2", "batched decode, 64 q / 8 KV heads, 16 x 32768 tokens, centroid, ratio 1/8 with bos+eos (4096 "
                 "tokens per sequence and head)",
           lambda: synth.batched_decode(cid=3, seq_lens=[32768] * 16), ops.Budget.ratio_budget(0.125, 1, 1),
           "centroid")
    yield ("ragged", "batched decode, 64 q / 8 KV heads, 16 x U[8192, 32768] tokens (8,409-30,271), centroid, "
                     "ratio 1/2 with bos+eos",
           lambda: synth.batched_decode(), ops.Budget.ratio_budget(0.5, 1, 1), "centroid")


def budget_sweep(a, dev, ceil=None):
    """Speedup over this build's dense kernel at every budget the pages use
    (with the gather ceiling of each 16-token-page record when `ceil` is
    given)."""
    import torch
    from block_sparse_attention_chunk_amd import ops, synth
    out = []
    log("budget sweep: replay-shaped layer, 1 x 29504 tokens, top-256 / top-512, both scorings")
    c1 = synth.replay_decode()
    t_dense = None
    for scoring in ("envelope", "centroid"):
        for k in (256, 512):
            log(f"  {scoring} top-{k}")
            b = DecodeBench(c1, ops.Budget.topk(k), scoring, dev, a.replicas_gib)
            m = b.measure_light(60, 5, t_dense=t_dense)
            t_dense = m["t_dense"]
            rec = record_light(f"replay-shaped decode, 1 x 29504 tokens, {scoring}, top-{k} pages", b, m,
                               f"{16 * k} tokens")
            out.append(attach_ceiling(rec, ceil, m["kv_bytes"]) if ceil else rec)
            del b
            torch.cuda.empty_cache()
    del c1
    log("budget sweep: variable chunks, 1 x 29504 tokens, token budgets 4096 / 8192 / 16384")
    c2 = synth.varchunk_decode()
    for tokens in (4096, 8192, 16384):
        log(f"  {tokens} tokens")
        b = ChunkedDecodeBench(c2, ops.Budget.token_budget(tokens), dev, a.replicas_gib)
        out.append(b.measure(60, 5))
        del b
        torch.cuda.empty_cache()
    del c2
    c2b = synth.varchunk_decode(seq_len=16384)
    b = ChunkedDecodeBench(c2b, ops.Budget.token_budget(16384), dev, a.replicas_gib)
    out.append(b.measure(60, 5))
    del b, c2b
    torch.cuda.empty_cache()
    log("budget sweep: 16 x U[8K, 32K] tokens, 64 q / 8 KV heads, seven ratios, both scorings")
    c3 = synth.batched_decode()
    ratios = [float(x) for x in a.sweep_ratios.split(",")] if a.sweep_ratios else synth.RATIOS
    t_dense = None
    for scoring, bos in (("centroid", 1), ("envelope", 0)):
        for ratio in ratios:
            log(f"  {scoring} ratio {ratio}")
            b = DecodeBench(c3, ops.Budget.ratio_budget(ratio, bos, 1), scoring, dev, a.replicas_gib)
            m = b.measure_light(30, 3, t_dense=t_dense)
            t_dense = m["t_dense"]
            rec = record_light(f"batched decode, 16 x U[8K, 32K], {scoring} (bos={bos}, eos=1), ratio {ratio}",
                               b, m, f"ratio {ratio}")
            out.append(attach_ceiling(rec, ceil, m["kv_bytes"]) if ceil else rec)
            del b
            torch.cuda.empty_cache()
    del c3
    return out


def calibration_copy(a, dev):
    """Profiling aid: one device-to-device copy of a known size, to scale the
    HBM byte counters of the same run."""
    if not a.calibration_copy_mib:
        return
    import torch
    n = a.calibration_copy_mib * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy of {n} bytes done")


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "bsa runs on one GPU: --gpus must be 1 (there is no multi-GPU path)"}))
        sys.exit(2)
    import torch
    from block_sparse_attention_chunk_amd import ops, synth
    dev = torch.device("cuda:0")

    recs = {}
    head_case = None
    for key, label, make, budget, scoring in decode_workloads(a.seq_len, a.budget, a.scoring):
        if a.only and key != a.only:
            continue
        if key != "headline" and (a.no_batched and not a.only):
            continue
        log(f"decode: {label}")
        case = make()
        b = DecodeBench(case, budget, scoring, dev, a.replicas_gib)
        steps = a.steps if key == "headline" else max(50, a.steps // 4)
        m = b.measure(steps, a.warmup if key == "headline" else 5, a.kernel_launches, a.samples)
        recs[key] = (record(label, b, m), m)
        if key == "headline":
            head_case = case
        del b
        torch.cuda.empty_cache()

    ceil, ceil_error = None, None
    if not a.no_ceiling:
        log("gather ceiling of the decode reads")
        try:
            ceil = GatherCeiling(torch, dev, a.replicas_gib)
            for key, (rec, mm) in recs.items():
                attach_ceiling(rec, ceil, mm["kv_bytes"])
        except (RuntimeError, OSError) as e:   # an auxiliary figure: the records stand without it
            ceil, ceil_error = None, str(e).splitlines()[0][:200]
            log(f"gather ceiling unavailable: {ceil_error}")
    if a.only:
        calibration_copy(a, dev)
        print(json.dumps(recs[a.only][0]), flush=True)
        return
    head, m = recs["headline"]
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
        "config": {"workload": head["workload"], "batch": 1, "seq_len": int(head_case.seq_lens[0]),
                   "q_heads": head_case.num_q_heads, "kv_heads": head_case.num_kv_heads,
                   "head_dim": head_case.head_dim, "page_size": head_case.page_size, "budget_tokens": a.budget,
                   "scoring": a.scoring, "splits": head["splits"], "cache_replicas": head["cache_replicas"],
                   "touched_bytes": head["touched_bytes"], "graph_replay": True},
        "effective_hbm_gbs": head["effective_hbm_gbs"],
        "effective_hbm_frac": head["effective_hbm_frac"],
        "us_per_step_median": head["us_per_step_median"],
        "us_per_step_p10": head["us_per_step_p10"],
        "us_per_step_p90": head["us_per_step_p90"],
        "roofline": {"bound": "hbm",
                     "kernel": "select_decode_kernel (the fused selection + attention launch of the step)",
                     "achieved": head["fused_kernel_selected_kv_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["fused_kernel_selected_kv_gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": m["kv_bytes"],
                     "launch_us": m["t_fused_kernel"] * 1e6},
        "practical_ceiling": ({"what": "bare gather of distinct random 4 KiB runs, the same bytes in one cold launch",
                               "gbs": head["gather_ceiling"]["gbs"],
                               "fused_kernel_frac": head["fused_kernel_of_ceiling"]}
                              if "gather_ceiling" in head else ({"unavailable": ceil_error} if ceil_error else None)),
        "headline": head,
    }
    if not a.no_batched:
        res["batched"] = [recs[k][0] for k in ("h1b16", "h2", "ragged")]
    if not a.no_sweep:
        res["budget_sweep"] = budget_sweep(a, dev, ceil)
    del ceil
    torch.cuda.empty_cache()
    attended = None
    if not a.no_prefill:
        log("router prefill: 131072 tokens")
        pc = synth.router_prefill()
        pb = PrefillBench(pc, dev, ops.BSA_ENVELOPE)
        res["prefill"] = pb.measure()
        attended = res["prefill"]["attended_blocks"]
        log("torch flash attention on the same prefill (outside reference)")
        res["prefill"]["torch_sdpa_flash_causal"] = torch_sdpa_causal(pc, dev, res["prefill"]["dense_causal_attn_ms"])
        del pb, pc
        torch.cuda.empty_cache()
        by_len = []
        for T in (32768, 65536):
            log(f"router prefill: {T} tokens")
            pc = synth.router_prefill(T=T, groups=max(4, T // 8192), tied_groups=tuple(range(3, max(4, T // 8192), 4)))
            pb = PrefillBench(pc, dev, ops.BSA_ENVELOPE)
            mm = pb.measure()
            by_len.append({k: mm[k] for k in ("workload", "tokens_per_s", "sparse_pipeline_ms", "tile_score_ms",
                                              "router_ms", "sparse_attn_ms", "dense_causal_attn_ms",
                                              "sparse_pipeline_vs_dense_attn", "triggered_tiles", "attn_mfma_frac")})
            del pb, pc
            torch.cuda.empty_cache()
        res["prefill_by_length"] = by_len
    if not a.no_layers:
        stacks = []
        for B, L in ((1, 32768), (16, 32768)):
            log(f"48-layer decode step, {B} sequence(s)")
            c = synth.replay_decode(seq_len=L) if B == 1 else synth.replay_decode(seq_len=L, batch=B)
            lb = LayerStackBench(c, ops.Budget.topk(256), "envelope", dev)
            stacks.append(lb.measure())
            del lb, c
            torch.cuda.empty_cache()
        res["layer_stack"] = stacks
    calibration_copy(a, dev)
    if not a.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(head_case, a.budget // 16, a.scoring, a.cpu_seconds, a.cpu_seconds_1t,
                                           attended)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
