"""Seeded synthetic inputs for block-sparse attention workloads.

This module only draws inputs.  It holds none of the method's arithmetic
(no metadata, scores, selection or attention): both the HIP path and the
oracle consume the bits it produces.  Every tensor comes from
``numpy.random.default_rng(SeedSequence([config_id, tensor_id]))`` and is
drawn in float32; bfloat16 inputs are the round-to-nearest-even bf16 of those
float32 values, stored as uint16 bit patterns.

Workloads (shapes from the pages' workloads; values synthetic):
  * tiny fp32 decode (1 x 1024 tokens, 8 q / 2 KV heads, d 64);
  * a decode layer shaped like the replay study's model on page 1 ("Sparse
    Attention for Web Agents", model line: GQA 32:4, head_dim 128) at the
    ~29.5k-token contexts of its "The comparison" section, with planted needle
    pages standing in for retrieval structure;
  * the same with variable 16-256-token chunks (page 1 method table, TSA row);
  * a batched paged decode shaped like a 64:8-head, d 128 model at 8K-32K tokens
    with the page-2 sparsity ratios;
  * a 131,072-token causal prefill with 28:4 heads for the router of page 3,
    with grouped needle blocks that make about a quarter of the tile cut-offs
    ambiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids of the seed sequence
T_K, T_V, T_Q, T_STRUCT, T_LENS, T_PERM, T_NEEDLE = range(7)

BF16, F32 = "bf16", "f32"


def rng(config_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(config_id), int(tensor_id)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


@dataclass
class DecodeCase:
    """Inputs of one decode step over a paged cache.

    k, v: [n_pages][H_kv][page_size][D] (uint16 bf16 bits, or float32);
    block_table: [B][max_pages] int32 (logical page -> physical page);
    seq_lens: [B] int32; q: [B][H_q][D].
    chunk_starts / num_chunks describe variable chunks ([B][max_chunks+1]
    token offsets, unused entries repeat the sequence length) or are None for
    fixed pages; chunk_len is [B][max_chunks] (0 past the last chunk).
    """
    name: str
    dtype: str
    k: np.ndarray
    v: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    q: np.ndarray
    page_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    chunk_starts: Optional[np.ndarray] = None
    num_chunks: Optional[np.ndarray] = None
    chunk_len: Optional[np.ndarray] = None
    info: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_chunks(self) -> int:
        return self.max_pages if self.chunk_starts is None else int(self.chunk_starts.shape[1] - 1)

    def n_chunks(self) -> np.ndarray:
        if self.chunk_starts is None:
            return ((self.seq_lens + self.page_size - 1) // self.page_size).astype(np.int32)
        return self.num_chunks.astype(np.int32)


def _paged_layout(cid: int, seq_lens, page_size: int, shuffle: bool = True):
    """Block table mapping every logical page of every sequence to a distinct
    physical page (a seeded permutation when shuffle)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    pages = (seq_lens + page_size - 1) // page_size
    total = int(pages.sum())
    max_pages = int(pages.max())
    perm = rng(cid, T_PERM).permutation(total) if shuffle else np.arange(total)
    bt = np.zeros((len(seq_lens), max_pages), dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, total



def make_decode(cid: int, *, batch: int, seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                page_size: int = 16, dtype: str = BF16, needles: int = 0, needle_gain: float = 0.3,
                outlier_channels: int = 0, outlier_scale: float = 8.0, channel_scale: Optional[tuple] = None,
                shuffle: bool = True, pad_value: Optional[float] = None, name: str = "decode") -> DecodeCase:
    """General paged decode case.

    Values: K, V, q ~ N(0, 1).  Optional structure, applied in this order:
      * needles > 0 (batch 1): that many distinct logical pages get +u_h added
        to every token's key (u_h ~ N(0, I) per KV head, same pages for every
        head);
      * outlier_channels: that many distinct channels per KV head scaled by
        outlier_scale;
      * channel_scale = (lo, hi): every (KV head, channel) of K and of V is
        scaled by its own U[lo, hi] factor (separate draws for K and V);
      * with needles, each q head = needle_gain * mean(needle keys of its KV
        head) + N(0, 1).
    Slots past a sequence's end in its last page hold N(0,1) noise, or
    pad_value when given (NaN there checks that no kernel reads them).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape[0] == batch
    bt, n_phys = _paged_layout(cid, seq_lens, page_size, shuffle)
    D, H, P = head_dim, num_kv_heads, page_size
    k = _normal(rng(cid, T_K), (n_phys, H, P, D))
    v = _normal(rng(cid, T_V), (n_phys, H, P, D))
    g_struct = rng(cid, T_STRUCT)
    info = {}
    needle_pages = None
    if needles:
        assert batch == 1
        n_pages = int((seq_lens[0] + P - 1) // P)
        gn = rng(cid, T_NEEDLE)
        needle_pages = np.sort(gn.choice(n_pages - 1, size=needles, replace=False)).astype(np.int32)
        u = _normal(gn, (H, D))
        phys = bt[0, needle_pages]
        k[phys] += u[None, :, None, :]
        info["needle_pages"] = needle_pages
    if outlier_channels:
        ch = np.stack([g_struct.choice(D, size=outlier_channels, replace=False) for _ in range(H)])
        for h in range(H):
            k[:, h, :, ch[h]] *= outlier_scale
        info["outlier_channels"] = ch
    if channel_scale is not None:
        lo, hi = channel_scale
        sk = g_struct.uniform(lo, hi, size=(H, D)).astype(np.float32)
        sv = g_struct.uniform(lo, hi, size=(H, D)).astype(np.float32)
        k *= sk[None, :, None, :]
        v *= sv[None, :, None, :]
    q = _normal(rng(cid, T_Q), (batch, num_q_heads, D))
    if needles:
        g = num_q_heads // H
        kn = k[bt[0, needle_pages]]                       # [needles][H][P][D], final key values
        mean = kn.transpose(1, 0, 2, 3).reshape(H, -1, D).mean(axis=1)
        q = q + needle_gain * np.repeat(mean, g, axis=0)[None]
    # tail slots of each sequence's last page
    for b in range(batch):
        L = int(seq_lens[b])
        if L % P:
            last = bt[b, L // P]
            if pad_value is not None:
                k[last, :, L % P:, :] = pad_value
                v[last, :, L % P:, :] = pad_value
    return DecodeCase(name=name, dtype=dtype, k=_store(k, dtype), v=_store(v, dtype), block_table=bt,
                      seq_lens=seq_lens, q=_store(q.astype(np.float32), dtype), page_size=P,
                      num_q_heads=num_q_heads, num_kv_heads=H, head_dim=D, info=info)


def variable_chunks(cid: int, seq_len: int, lo: int = 16, hi: int = 256):
    """Chunk lengths drawn uniformly from the integers [lo, hi] until they
    cover seq_len; the last one is clipped.  Returns chunk starts (n+1)."""
    g = rng(cid, T_LENS)
    starts = [0]
    while starts[-1] < seq_len:
        starts.append(min(seq_len, starts[-1] + int(g.integers(lo, hi + 1))))
    return np.asarray(starts, dtype=np.int32)


def with_chunks(case: DecodeCase, starts_per_seq) -> DecodeCase:
    """Attach variable chunk boundaries (one start array per sequence)."""
    B = case.batch
    n = np.array([len(s) - 1 for s in starts_per_seq], dtype=np.int32)
    mc = int(n.max())
    cs = np.zeros((B, mc + 1), dtype=np.int32)
    cl = np.zeros((B, mc), dtype=np.int32)
    for b, s in enumerate(starts_per_seq):
        s = np.asarray(s, dtype=np.int32)
        cs[b, :len(s)] = s
        cs[b, len(s):] = s[-1]
        cl[b, :len(s) - 1] = np.diff(s)
    case.chunk_starts, case.num_chunks, case.chunk_len = cs, n, cl
    return case


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

def tiny_decode(cid: int = 0) -> DecodeCase:
    """1 sequence x 1024 tokens, 8 q / 2 KV heads, d 64, fp32, 16-token pages;
    K, V, q ~ N(0, 1)."""
    return make_decode(cid, batch=1, seq_lens=[1024], num_q_heads=8, num_kv_heads=2, head_dim=64, dtype=F32,
                       name="tiny-decode-fp32")


def replay_decode(cid: int = 1, seq_len: int = 29504, batch: int = 1) -> DecodeCase:
    """Decode layer with 32 q / 4 KV heads, d 128, bf16, 16-token pages.
    K ~ N(0,1) with 24 planted needle pages (+u_h) and 4 outlier channels x8
    per KV head; V ~ N(0,1); q = 0.3 x mean(needle keys) + N(0,1).
    batch > 1 stacks independent sequences of the same length (no needles)."""
    if batch == 1:
        return make_decode(cid, batch=1, seq_lens=[seq_len], num_q_heads=32, num_kv_heads=4, head_dim=128,
                           dtype=BF16, needles=24, needle_gain=0.3, outlier_channels=4, outlier_scale=8.0,
                           name=f"replay-decode-{seq_len}")
    return make_decode(cid, batch=batch, seq_lens=[seq_len] * batch, num_q_heads=32, num_kv_heads=4,
                       head_dim=128, dtype=BF16, outlier_channels=4, outlier_scale=8.0,
                       name=f"replay-decode-{seq_len}x{batch}")


def varchunk_decode(cid: int = 2, seq_len: int = 29504) -> DecodeCase:
    """The replay-shaped decode with chunk lengths drawn from U[16, 256]."""
    case = replay_decode(cid, seq_len)
    case.name = f"varchunk-decode-{seq_len}"
    return with_chunks(case, [variable_chunks(cid, seq_len)])


def batched_decode(cid: int = 3, batch: int = 16, lo: int = 8192, hi: int = 32768, num_q_heads: int = 64,
                   num_kv_heads: int = 8, head_dim: int = 128, seq_lens=None) -> DecodeCase:
    """Batched paged decode: lengths ~ U[lo, hi] (integers), 64 q / 8 KV
    heads, d 128, bf16, shuffled block table; K and V scaled per (KV head,
    channel) by U[0.5, 4]; q ~ N(0,1)."""
    if seq_lens is None:
        seq_lens = rng(cid, T_LENS).integers(lo, hi + 1, size=batch)
    return make_decode(cid, batch=batch, seq_lens=seq_lens, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, dtype=BF16, channel_scale=(0.5, 4.0),
                       name=f"batched-decode-{batch}x[{lo},{hi}]")


RATIOS = (0.5, 0.375, 0.25, 0.125, 0.0625, 0.03125, 0.015625)


@dataclass
class PrefillCase:
    """Inputs of one causal prefill: Q [T][H_q][D], K/V [T][H_kv][D]
    (token-major, uint16 bf16 bits), key blocks of `block` tokens and query
    tiles of `tile` rows."""
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block: int
    tile: int
    info: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])


def router_prefill(cid: int = 4, T: int = 131072, num_q_heads: int = 28, num_kv_heads: int = 4,
                   head_dim: int = 128, block: int = 64, k: int = 32, groups: int = 16,
                   tied_groups=(3, 7, 11, 15), gain: float = 0.3, twin_gain: float = 0.15, alpha: float = 2.0,
                   rms_heads=(0, 1)) -> PrefillCase:
    """Causal prefill with grouped needle blocks, per KV head h:
      1. tiles are split into `groups` contiguous groups; each group gets a
         direction u ~ N(0, I);
      2. each group owns k needle blocks drawn without reuse (per head) from
         the blocks every tile of the group can see, [0, max(k+1, first tile));
      3. needle keys become gain*u + sqrt(1-gain^2)*K;
      4. in the tied groups, k-1 strong needles plus a twin pair at twin_gain,
         the second twin = first twin + 1e-3*N(0,1);
      5. queries of a tile: (N(0,1) + alpha*u_group) / sqrt(1+alpha^2).
    Then the KV heads in rms_heads and their query groups are RMS-normalised
    (x / sqrt(mean x^2 + 1e-6)).  V ~ N(0,1)."""
    D, H, g = head_dim, num_kv_heads, num_q_heads // num_kv_heads
    n_tiles = T // block
    per_group = max(1, n_tiles // groups)
    K = _normal(rng(cid, T_K), (T, H, D))
    V = _normal(rng(cid, T_V), (T, H, D))
    Q = _normal(rng(cid, T_Q), (T, num_q_heads, D))
    gn = rng(cid, T_NEEDLE)
    info = {"needles": {}, "per_group": per_group, "n_groups": 0}
    n_groups = (n_tiles + per_group - 1) // per_group
    info["n_groups"] = n_groups
    c2 = np.float32(np.sqrt(1.0 - gain * gain))
    for h in range(H):
        used = np.zeros(n_tiles, dtype=bool)
        for gi in range(n_groups):
            u = _normal(gn, (D,))
            first_tile = gi * per_group
            pool_hi = min(n_tiles, max(k + 1, first_tile))
            tied = gi in tied_groups
            want = k + 1 if tied else k
            pool = np.flatnonzero(~used[:pool_hi])
            want = min(want, len(pool))
            chosen = np.sort(gn.choice(pool, size=want, replace=False)) if want else np.zeros(0, dtype=np.int64)
            used[chosen] = True
            strong = chosen if not tied else chosen[:-2]
            for b in strong:
                sl = slice(b * block, (b + 1) * block)
                K[sl, h, :] = gain * u[None, :] + c2 * K[sl, h, :]
            if tied and want >= 2:
                b1, b2 = chosen[-2], chosen[-1]
                ct = np.float32(np.sqrt(1.0 - twin_gain * twin_gain))
                s1, s2 = slice(b1 * block, (b1 + 1) * block), slice(b2 * block, (b2 + 1) * block)
                K[s1, h, :] = twin_gain * u[None, :] + ct * K[s1, h, :]
                K[s2, h, :] = K[s1, h, :] + np.float32(1e-3) * _normal(gn, (block, D))
            info["needles"][(h, gi)] = chosen
            rows = slice(first_tile * block, min(T, (first_tile + per_group) * block))
            Q[rows, h * g:(h + 1) * g, :] = (Q[rows, h * g:(h + 1) * g, :] + alpha * u) / np.float32(
                np.sqrt(1.0 + alpha * alpha))
    for h in rms_heads:
        if h >= H:
            continue
        kh = K[:, h, :]
        K[:, h, :] = kh / np.sqrt(np.mean(kh * kh, axis=-1, keepdims=True) + np.float32(1e-6))
        qh = Q[:, h * g:(h + 1) * g, :]
        Q[:, h * g:(h + 1) * g, :] = qh / np.sqrt(np.mean(qh * qh, axis=-1, keepdims=True) + np.float32(1e-6))
    return PrefillCase(name=f"router-prefill-{T}", q=f32_to_bf16_bits(Q), k=f32_to_bf16_bits(K),
                       v=f32_to_bf16_bits(V), num_q_heads=num_q_heads, num_kv_heads=H, head_dim=D, block=block,
                       tile=block, info=info)
