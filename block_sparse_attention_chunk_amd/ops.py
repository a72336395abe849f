"""Python binding of libbsa with the C ABI's entry-point names.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step runs in the library's HIP kernels.  Outputs are
allocated with torch when not given.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional

import torch

from . import _abi
from ._abi import (BSA_BF16, BSA_BUDGET_RATIO, BSA_BUDGET_TOKENS, BSA_BUDGET_TOPK, BSA_CENTROID, BSA_ENVELOPE,
                   BSA_F32, BSA_META_CENTROID, BSA_META_ENVELOPE)

__all__ = ["upload", "KVCache", "Chunks", "Meta", "Budget", "build_chunk_meta", "score_chunks", "select_topk",
           "select_topk_router", "sparse_attn_decode", "sparse_attn_tile_prefill", "tile_prefill_workspace_bytes",
           "decode_workspace_bytes", "decode_step", "decode_step_workspace_bytes", "select_attn_decode",
           "router_workspace_bytes", "decode_num_splits"]


def upload(x, device="cuda") -> torch.Tensor:
    """Copy a host array to the device: uint16 arrays hold bfloat16 bit patterns."""
    import numpy as np
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(x).to(device)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class KVCache:
    """A paged K/V cache in device memory.

    paged layout:       k, v [n_pages][H_kv][page_size][D] (any strides, the
                        same for both), block_table [B][max_pages]
    token-major layout: k, v [T][H_kv][D] in blocks of page_size tokens (batch 1,
                        block_table None)
    """
    k: torch.Tensor
    v: Optional[torch.Tensor]
    seq_lens: torch.Tensor
    page_size: int
    block_table: Optional[torch.Tensor] = None
    token_major: bool = False
    max_pages: Optional[int] = None

    def __post_init__(self):
        k = self.k
        # element strides are taken from the tensors, so K and V may be views
        # into one buffer (e.g. [n_pages][H_kv][2][page_size][D], K and V of a
        # page next to each other); both must share them
        if self.v is not None and tuple(self.v.stride()) != tuple(k.stride()):
            raise ValueError("k and v must have the same strides")
        if k.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
        if self.token_major:
            T, H, D = k.shape
            self.num_kv_heads, self.head_dim = H, D
            self.strides = (self.page_size * k.stride(0), k.stride(1), k.stride(0))
            if self.max_pages is None:
                self.max_pages = (T + self.page_size - 1) // self.page_size
        else:
            _, H, P, D = k.shape
            assert P == self.page_size
            self.num_kv_heads, self.head_dim = H, D
            self.strides = (k.stride(0), k.stride(1), k.stride(2))
            if self.max_pages is None:
                self.max_pages = int(self.block_table.shape[1])
        self.batch = int(self.seq_lens.shape[0])
        self.dtype = _dtype_code(k)

    def struct(self) -> _abi.bsa_kv:
        return _abi.bsa_kv(self.k.data_ptr(), None if self.v is None else self.v.data_ptr(), self.strides[0],
                           self.strides[1],
                           self.strides[2], None if self.block_table is None else self.block_table.data_ptr(),
                           self.seq_lens.data_ptr(), self.batch, self.num_kv_heads, self.head_dim, self.page_size,
                           self.max_pages, self.dtype)


@dataclass
class Chunks:
    """Variable chunk boundaries: starts [B][max_chunks+1], num [B] (int32)."""
    starts: torch.Tensor
    num: torch.Tensor

    @property
    def max_chunks(self) -> int:
        return int(self.starts.shape[1] - 1)

    def struct(self) -> _abi.bsa_chunks:
        return _abi.bsa_chunks(self.starts.data_ptr(), self.num.data_ptr(), self.max_chunks)


def _chunks_struct(chunks: Optional[Chunks]):
    return None if chunks is None else ctypes.byref(chunks.struct())


def _max_chunks(kv: KVCache, chunks: Optional[Chunks]) -> int:
    return kv.max_pages if chunks is None else chunks.max_chunks


@dataclass
class Meta:
    kmin: Optional[torch.Tensor] = None
    kmax: Optional[torch.Tensor] = None
    centroid: Optional[torch.Tensor] = None

    def struct(self) -> _abi.bsa_meta:
        return _abi.bsa_meta(None if self.kmin is None else self.kmin.data_ptr(),
                             None if self.kmax is None else self.kmax.data_ptr(),
                             None if self.centroid is None else self.centroid.data_ptr())


@dataclass
class Budget:
    mode: int
    top_k: int = 0
    tokens: int = 0
    bos: int = 0
    eos: int = 0
    ratio: float = 0.0

    @staticmethod
    def topk(k: int) -> "Budget":
        return Budget(BSA_BUDGET_TOPK, top_k=k)

    @staticmethod
    def token_budget(tokens: int) -> "Budget":
        return Budget(BSA_BUDGET_TOKENS, tokens=tokens)

    @staticmethod
    def ratio_budget(ratio: float, bos: int, eos: int) -> "Budget":
        return Budget(BSA_BUDGET_RATIO, ratio=ratio, bos=bos, eos=eos)

    def struct(self) -> _abi.bsa_budget:
        return _abi.bsa_budget(self.mode, self.top_k, self.tokens, self.bos, self.eos, self.ratio)

    def max_selected(self, max_chunks: int) -> int:
        """bsa_select_max_count: the largest selection a row of max_chunks
        candidates can keep under this budget (the size of max_sel)."""
        n = int(_abi.lib().bsa_select_max_count(ctypes.byref(self.struct()), int(max_chunks)))
        _abi.check(min(n, 0), "bsa_select_max_count")
        return n


def build_chunk_meta(kv: KVCache, chunks: Optional[Chunks] = None, which: int = BSA_META_ENVELOPE | BSA_META_CENTROID,
                     meta: Optional[Meta] = None) -> Meta:
    """bsa_build_chunk_meta: per-chunk kmin / kmax (cache dtype) and centroid (fp32),
    each [B][H_kv][max_chunks][D]."""
    mc = _max_chunks(kv, chunks)
    shape = (kv.batch, kv.num_kv_heads, mc, kv.head_dim)
    dev = kv.k.device
    if meta is None:
        meta = Meta()
        if which & BSA_META_ENVELOPE:
            meta.kmin = torch.empty(shape, dtype=kv.k.dtype, device=dev)
            meta.kmax = torch.empty(shape, dtype=kv.k.dtype, device=dev)
        if which & BSA_META_CENTROID:
            meta.centroid = torch.empty(shape, dtype=torch.float32, device=dev)
    L = _abi.lib()
    rc = L.bsa_build_chunk_meta(ctypes.byref(kv.struct()), _chunks_struct(chunks), ctypes.byref(meta.struct()),
                                which, _stream(dev))
    _abi.check(rc, "bsa_build_chunk_meta")
    return meta


def update_chunk_meta(kv: KVCache, meta: Meta, which: int = BSA_META_ENVELOPE | BSA_META_CENTROID,
                      from_len: Optional[torch.Tensor] = None, max_touched: int = 1,
                      chunks: Optional[Chunks] = None) -> Meta:
    """bsa_update_chunk_meta: refresh the chunks touched by tokens at positions
    >= from_len[b] (the last chunk when from_len is None) in place."""
    L = _abi.lib()
    rc = L.bsa_update_chunk_meta(ctypes.byref(kv.struct()), _chunks_struct(chunks), ctypes.byref(meta.struct()), which,
                                 _ptr(from_len), int(max_touched), _stream(kv.k.device))
    _abi.check(rc, "bsa_update_chunk_meta")
    return meta


def score_chunks(q: torch.Tensor, kv: KVCache, meta: Meta, kind: int, rows_per_query: int = 1, causal: bool = False,
                 chunks: Optional[Chunks] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsa_score_chunks.  Decode: q [B][H_q][D] -> [B][H_kv][max_chunks].
    Tiles: q [T][H_q][D] -> [ceil(T/R)][H_kv][max_chunks]."""
    mc = _max_chunks(kv, chunks)
    rows = q.shape[0]
    n_out = rows if rows_per_query == 1 else (rows + rows_per_query - 1) // rows_per_query
    if out is None:
        out = torch.empty((n_out, kv.num_kv_heads, mc), dtype=torch.float32, device=q.device)
    L = _abi.lib()
    rc = L.bsa_score_chunks(_ptr(q), q.shape[1], rows, rows_per_query, ctypes.byref(kv.struct()),
                            _chunks_struct(chunks), ctypes.byref(meta.struct()), kind, int(bool(causal)), _ptr(out),
                            _stream(q.device))
    _abi.check(rc, "bsa_score_chunks")
    return out


def select_topk(scores: torch.Tensor, kv: KVCache, budget: Budget, chunks: Optional[Chunks] = None,
                max_sel: Optional[int] = None, sel_idx: Optional[torch.Tensor] = None,
                sel_count: Optional[torch.Tensor] = None):
    """bsa_select_topk -> (sel_idx [B][H_kv][max_sel] ascending, -1 padded; sel_count [B][H_kv])."""
    mc = _max_chunks(kv, chunks)
    if max_sel is None:
        max_sel = budget.max_selected(mc)
    dev = scores.device
    if sel_idx is None:
        sel_idx = torch.empty((kv.batch, kv.num_kv_heads, max_sel), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((kv.batch, kv.num_kv_heads), dtype=torch.int32, device=dev)
    L = _abi.lib()
    rc = L.bsa_select_topk(_ptr(scores), ctypes.byref(kv.struct()), _chunks_struct(chunks),
                           ctypes.byref(budget.struct()), _ptr(sel_idx), _ptr(sel_count), max_sel, _stream(dev))
    _abi.check(rc, "bsa_select_topk")
    return sel_idx, sel_count


def router_workspace_bytes(num_tiles: int, num_kv_heads: int, k: int, rho: int) -> int:
    return int(_abi.lib().bsa_router_workspace_bytes(num_tiles, num_kv_heads, k, rho))


def select_topk_router(tile_scores: torch.Tensor, k: int, rho: int, quantile: float = 0.25,
                       fixed_threshold: Optional[float] = None, causal: bool = True,
                       workspace: Optional[torch.Tensor] = None) -> dict:
    """bsa_select_topk_router -> dict(kv_idx, sigma, sigma_bar, triggered, threshold)."""
    nt, H, nb = tile_scores.shape
    dev = tile_scores.device
    kv_idx = torch.empty((nt, H, rho * k), dtype=torch.int32, device=dev)
    sigma = torch.empty((nt, H), dtype=torch.float32, device=dev)
    sigma_bar = torch.empty((nt,), dtype=torch.float32, device=dev)
    trig = torch.empty((nt,), dtype=torch.uint8, device=dev)
    thr = torch.empty((1,), dtype=torch.float32, device=dev)
    need = router_workspace_bytes(nt, H, k, rho)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L = _abi.lib()
    rc = L.bsa_select_topk_router(_ptr(tile_scores), nt, H, nb, int(bool(causal)), k, rho, float(quantile),
                                  float("nan") if fixed_threshold is None else float(fixed_threshold), _ptr(kv_idx),
                                  _ptr(sigma), _ptr(sigma_bar), _ptr(trig), _ptr(thr), _ptr(workspace), ws_bytes,
                                  _stream(dev))
    _abi.check(rc, "bsa_select_topk_router")
    return {"kv_idx": kv_idx, "sigma": sigma, "sigma_bar": sigma_bar, "triggered": trig, "threshold": thr}


def decode_num_splits(kv: KVCache, num_q_heads: int, max_items: int, num_splits: int = 0) -> int:
    return int(_abi.lib().bsa_decode_num_splits(ctypes.byref(kv.struct()), num_q_heads, max_items, num_splits))


def decode_workspace_bytes(kv: KVCache, num_q_heads: int, max_items: int, num_splits: int = 0) -> int:
    return int(_abi.lib().bsa_decode_workspace_bytes(ctypes.byref(kv.struct()), num_q_heads, max_items, num_splits))


def sparse_attn_decode(q: torch.Tensor, kv: KVCache, sel_idx: Optional[torch.Tensor] = None,
                       sel_count: Optional[torch.Tensor] = None, chunks: Optional[Chunks] = None,
                       scale: Optional[float] = None, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsa_sparse_attn_decode: q [B][H_q][D] -> out [B][H_q][D] float32; sel_idx None = dense.
    out=PARTIALS leaves the split partials in the workspace (see decode_merge).
    With automatic splits (num_splits=0), out given and a large batch of
    16-token pages, the attention runs on the balanced schedule."""
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    elif out is PARTIALS:
        out = None
    max_sel = 0 if sel_idx is None else int(sel_idx.shape[2])
    items = max_sel if sel_idx is not None else _max_chunks(kv, chunks)
    need = decode_workspace_bytes(kv, Hq, items, num_splits)
    if workspace is None and need:
        workspace = torch.zeros((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L = _abi.lib()
    rc = L.bsa_sparse_attn_decode(_ptr(q), Hq, ctypes.byref(kv.struct()), _chunks_struct(chunks), _ptr(sel_idx),
                                  _ptr(sel_count), max_sel, float(scale), num_splits, _ptr(out), _ptr(workspace),
                                  ws_bytes, _stream(q.device))
    _abi.check(rc, "bsa_sparse_attn_decode")
    return out


PARTIALS = object()   # out=PARTIALS: skip the split merge, keep the partials in the workspace


def decode_merge(workspace: torch.Tensor, batch: int, num_q_heads: int, head_dim: int, num_splits: int,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsa_decode_merge: the split partials in `workspace` -> out [B][H_q][D] float32."""
    if out is None:
        out = torch.empty((batch, num_q_heads, head_dim), dtype=torch.float32, device=workspace.device)
    rc = _abi.lib().bsa_decode_merge(_ptr(workspace), batch, num_q_heads, head_dim, num_splits, _ptr(out),
                                     _stream(workspace.device))
    _abi.check(rc, "bsa_decode_merge")
    return out


def select_attn_decode(q: torch.Tensor, kv: KVCache, scores: torch.Tensor, budget: Budget,
                       scale: Optional[float] = None, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, sel_idx: Optional[torch.Tensor] = None,
                       sel_count: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsa_select_attn_decode: selection + attention in one launch (16-token
    pages).  q [B][H_q][D], scores [B][H_kv][max_pages] -> out [B][H_q][D]
    float32; sel_idx / sel_count, when given, receive the kept list.  With
    automatic splits on a large batch the library runs the selection kernel
    and the balanced attention instead (the same bits as the two calls)."""
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    elif out is PARTIALS:
        out = None
    K = budget.max_selected(kv.max_pages)
    need = decode_workspace_bytes(kv, Hq, K, num_splits)
    if workspace is None and need:
        workspace = torch.zeros((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    max_sel = 0 if sel_idx is None else int(sel_idx.shape[2])
    L = _abi.lib()
    rc = L.bsa_select_attn_decode(_ptr(q), Hq, ctypes.byref(kv.struct()), _ptr(scores),
                                  ctypes.byref(budget.struct()), float(scale), num_splits, _ptr(out), _ptr(sel_idx),
                                  _ptr(sel_count), max_sel, _ptr(workspace), ws_bytes, _stream(q.device))
    _abi.check(rc, "bsa_select_attn_decode")
    return out


def decode_step_workspace_bytes(kv: KVCache, num_q_heads: int, budget: Budget, num_splits: int = 0) -> int:
    return int(_abi.lib().bsa_decode_step_workspace_bytes(ctypes.byref(kv.struct()), num_q_heads,
                                                          ctypes.byref(budget.struct()), num_splits))


def decode_step(q: torch.Tensor, kv: KVCache, meta: Meta, kind: int, budget: Budget, scale: Optional[float] = None,
                num_splits: int = 0, out: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, sel_idx: Optional[torch.Tensor] = None,
                sel_count: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsa_decode_step: chunk scores, selection, attention and split merge of
    one decode step (16-token pages) in one call.  q [B][H_q][D] -> out
    [B][H_q][D] float32; scores / sel_idx / sel_count, when given, receive
    the chunk scores and the kept list."""
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    need = decode_step_workspace_bytes(kv, Hq, budget, num_splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    max_sel = 0 if sel_idx is None else int(sel_idx.shape[2])
    rc = _abi.lib().bsa_decode_step(_ptr(q), Hq, ctypes.byref(kv.struct()), ctypes.byref(meta.struct()), kind,
                                    ctypes.byref(budget.struct()), float(scale), num_splits, _ptr(out), _ptr(scores),
                                    _ptr(sel_idx), _ptr(sel_count), max_sel, _ptr(workspace), ws_bytes,
                                    _stream(q.device))
    _abi.check(rc, "bsa_decode_step")
    return out


def tile_prefill_workspace_bytes(kv: KVCache, num_rows: int) -> int:
    return int(_abi.lib().bsa_tile_prefill_workspace_bytes(ctypes.byref(kv.struct()), num_rows))


def sparse_attn_tile_prefill(q: torch.Tensor, kv: KVCache, kv_idx: Optional[torch.Tensor] = None, tile_rows: int = 64,
                             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bsa_sparse_attn_tile_prefill: q [T][H_q][D] bf16 -> out [T][H_q][D] float32;
    kv_idx [n_tiles][H_kv][stride] (-1 padded) or None (dense causal).  The
    workspace (an fp16 copy of V) is allocated when not given."""
    T, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty((max(tile_prefill_workspace_bytes(kv, T), 16),), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    stride = 0 if kv_idx is None else int(kv_idx.shape[-1])
    L = _abi.lib()
    rc = L.bsa_sparse_attn_tile_prefill(_ptr(q), Hq, T, ctypes.byref(kv.struct()), tile_rows, _ptr(kv_idx), stride,
                                        float(scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(q.device))
    _abi.check(rc, "bsa_sparse_attn_tile_prefill")
    return out
