"""Helpers for the GPU-vs-oracle parity tests: run the HIP path through the
C ABI, run the oracle on the same input bits, and compare stage by stage."""
from __future__ import annotations

import math
import sys
import time

import numpy as np

import oracle
from block_sparse_attention_chunk_amd import synth

# Tolerances (the parity gates; denominators D = sum_d |term_d| of the oracle's dot product)
SCORE_REL = 1e-4          # |s_gpu - s_oracle| <= 1e-4 * D
BAND_REL = 5e-4           # selection may differ only within +-5e-4 * D of the cut midpoint
ATTN_ABS = {"bf16": 2e-3, "f32": 1e-5}


def unequal_rows_case(cid: int, dtype: str, head_dim: int, sel_seed: int, num_q_heads: int = 8):
    """8 sequences x 2 KV heads (num_q_heads q heads) with hand-made selections of very
    unequal sizes, in a kept-list capacity of 4096 pages: one row keeps all
    2048 pages of a 32K sequence, two rows keep nothing, several keep one page,
    and partial last pages occur.  Returns (case, sel_idx, sel_count)."""
    lens = [32768, 600, 100, 20, 5000, 16, 1, 3000]
    counts = [[2048, 0], [38, 1], [0, 7], [2, 1], [313, 200], [1, 0], [1, 1], [188, 50]]
    case = synth.make_decode(cid, batch=8, seq_lens=lens, num_q_heads=num_q_heads, num_kv_heads=2,
                             head_dim=head_dim, dtype=dtype, name=f"unequal-rows-{dtype}-{head_dim}-{num_q_heads}q")
    gen = np.random.default_rng(sel_seed)
    sel = np.full((8, 2, 4096), -1, dtype=np.int32)
    cnt = np.array(counts, dtype=np.int32)
    for b in range(8):
        pages = (lens[b] + 15) // 16
        for h in range(2):
            sel[b, h, :cnt[b, h]] = np.sort(gen.choice(pages, size=cnt[b, h], replace=False))
    return case, sel, cnt


def log(msg):
    print(f"[parity] {time.strftime('%H:%M:%S')} {msg}", flush=True)
    sys.stdout.flush()


def gpu_kv(case, dev):
    import torch  # noqa: F401
    from block_sparse_attention_chunk_amd import ops
    kv = ops.KVCache(ops.upload(case.k, dev), ops.upload(case.v, dev), ops.upload(case.seq_lens, dev),
                     case.page_size, ops.upload(case.block_table, dev))
    chunks = None
    if case.chunk_starts is not None:
        chunks = ops.Chunks(ops.upload(case.chunk_starts, dev), ops.upload(case.num_chunks, dev))
    return kv, chunks


def oracle_cache(case):
    return oracle.PagedCache(case.k, case.v, case.block_table, case.seq_lens, case.page_size, case.num_kv_heads,
                             case.head_dim)


def oracle_select(scores, case, budget):
    from block_sparse_attention_chunk_amd import ops
    n = case.n_chunks()
    chunk_len = case.chunk_len
    if budget.mode == ops.BSA_BUDGET_TOKENS and chunk_len is None:
        chunk_len = np.zeros((case.batch, case.max_chunks), np.int32)
        for b in range(case.batch):
            L = int(case.seq_lens[b])
            for c in range(int(n[b])):
                chunk_len[b, c] = min(case.page_size, L - c * case.page_size)
    mode = {ops.BSA_BUDGET_TOPK: oracle.TOPK, ops.BSA_BUDGET_TOKENS: oracle.TOKENS,
            ops.BSA_BUDGET_RATIO: oracle.RATIO}[budget.mode]
    # rows as wide as the whole candidate list: the oracle's buffer size owes
    # nothing to the library's sizing rule; counts are compared, not widths
    return oracle.select(scores, n, mode, top_k=budget.top_k, tokens=budget.tokens, ratio=budget.ratio,
                         bos=budget.bos, eos=budget.eos, chunk_len=chunk_len, max_sel=case.max_chunks)


def check_scores(gpu, ref, den, n_chunks, what):
    worst = 0.0
    for b in range(ref.shape[0]):
        n = int(n_chunks[b])
        d = np.abs(gpu[b, :, :n].astype(np.float64) - ref[b, :, :n])
        r = d / np.maximum(den[b, :, :n], 1e-30)
        worst = max(worst, float(r.max()))
        assert np.all(d <= SCORE_REL * den[b, :, :n] + 1e-30), f"{what}: score error {r.max():.3g} D"
        assert np.all(np.isneginf(gpu[b, :, n:])), f"{what}: padding chunks must be -inf"
    return worst


def check_band(sel_gpu, cnt_gpu, sel_ref, cnt_ref, scores_ref, den, n_chunks, forced=(), exact_count=True):
    """Band rule: every candidate further than BAND_REL*D from the cut midpoint
    is kept by both or by neither; returns the number of in-band differences."""
    diffs = 0
    B, H = cnt_ref.shape
    for b in range(B):
        n = int(n_chunks[b])
        for h in range(H):
            g = set(sel_gpu[b, h, :cnt_gpu[b, h]].tolist())
            r = set(sel_ref[b, h, :cnt_ref[b, h]].tolist())
            if exact_count:
                assert cnt_gpu[b, h] == cnt_ref[b, h], (b, h, cnt_gpu[b, h], cnt_ref[b, h])
            if g == r:
                continue
            s = scores_ref[b, h, :n]
            fixed = {0 if f == "bos" else n - 1 for f in forced}
            cand = [c for c in range(n) if c not in fixed]
            kept = [s[c] for c in cand if c in r]
            dropped = [s[c] for c in cand if c not in r]
            assert kept and dropped, (b, h)
            mid = 0.5 * (min(kept) + max(dropped))
            for c in (g ^ r):
                assert abs(s[c] - mid) <= BAND_REL * den[b, h, c], (
                    f"chunk {c} of (b={b}, h={h}) differs outside the band: |s-mid|={abs(s[c]-mid):.3g}, "
                    f"D={den[b, h, c]:.3g}")
            diffs += len(g ^ r)
    return diffs


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
