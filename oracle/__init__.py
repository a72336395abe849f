"""fp64 CPU oracle for query-aware block-sparse attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library; both sides only read the same seeded
input bits produced by ``block_sparse_attention_chunk_amd.synth``.

All arithmetic lives in ``bsa_oracle.c`` (plain double-precision loops).  This
module only converts inputs to float64 (bf16 bits widen exactly) and marshals
pointers.  Every function cites the page section it follows; see the C file
for the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation tests point this at a deliberately broken build of the oracle.
_LIB_OVERRIDE = os.environ.get("BSA_ORACLE_LIB")

ENVELOPE, CENTROID = 0, 1
TOPK, TOKENS, RATIO = 0, 1, 2

# Parity status of each oracle function (pinned = checked against something
# other than itself by the CPU tests in tests/test_oracle_pins.py).
PARITY = {
    "chunk_meta": "pinned",
    "score_decode": "pinned",
    "select": "pinned",
    "decode_attn": "pinned",
    "tile_scores": "pinned",
    "router": "pinned",
    "quantile": "pinned",
    "tile_attn": "pinned",
}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("stride_page", ctypes.c_int64), ("stride_head", ctypes.c_int64),
                ("stride_token", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.orc_chunk_meta.argtypes = [P, P, P, i32, P, P, P]
        lib.orc_score_decode.argtypes = [P, i32, P, P, P, i32, P, P, P, i32, P, P, P]
        lib.orc_select.argtypes = [P, i32, i32, i32, P, P, i32, i32, i64, f64, i32, i32, P, P, i32]
        lib.orc_select.restype = ctypes.c_int
        lib.orc_decode_attn.argtypes = [P, i32, P, P, P, i32, P, P, i32, f64, P]
        lib.orc_tile_scores.argtypes = [P, i32, i32, i32, i32, P, P, P, i32, i32, i32, i32, i32, P, i32, P, P]
        lib.orc_quantile.argtypes = [P, i32, f64]
        lib.orc_quantile.restype = f64
        lib.orc_router.argtypes = [P, i32, i32, i32, P, i32, i32, f64, i32, f64, P, P, P, P, P, P]
        lib.orc_tile_attn.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, i32, f64, P, i32, P]
        _lib = lib
    return _lib


def _gomp():
    _load()                      # the oracle library links the OpenMP runtime
    return ctypes.CDLL("libgomp.so.1")


def set_threads(n: int) -> None:
    """Number of OpenMP threads the oracle's parallel loops use from now on."""
    _gomp().omp_set_num_threads(int(n))


def max_threads() -> int:
    """Threads the oracle's next parallel loop will use."""
    return int(_gomp().omp_get_max_threads())


def to_f64(x: np.ndarray) -> np.ndarray:
    """Widen an input to float64: uint16 arrays hold bfloat16 bit patterns
    (exact widening), float32 / float64 arrays are converted exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        with np.errstate(invalid="ignore"):
            return np.ascontiguousarray((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


class PagedCache:
    """A paged K/V cache widened to float64.

    ``k``/``v``: arrays whose element (page, head, slot, dim) sits at
    page*stride_page + head*stride_head + slot*stride_token + dim.  By default
    they are [n_pages][H_kv][page_size][D]; a token-major [T][H_kv][D] cache
    is described with page_size = block and strides (block*H_kv*D, D, H_kv*D).
    """

    def __init__(self, k, v, block_table, seq_lens, page_size, num_kv_heads, head_dim, strides=None,
                 max_pages=None):
        self.k = to_f64(k)
        self.v = to_f64(v) if v is not None else None
        self.block_table = _i32(block_table)
        self.seq_lens = _i32(seq_lens)
        self.batch = int(self.seq_lens.shape[0])
        self.num_kv_heads, self.head_dim, self.page_size = int(num_kv_heads), int(head_dim), int(page_size)
        if strides is None:
            strides = (num_kv_heads * page_size * head_dim, page_size * head_dim, head_dim)
        self.strides = tuple(int(s) for s in strides)
        if max_pages is None:
            max_pages = self.block_table.shape[1]
        self.max_pages = int(max_pages)

    def _struct(self):
        return _Cache(self.k.ctypes.data, None if self.v is None else self.v.ctypes.data,
                      self.strides[0], self.strides[1], self.strides[2],
                      _p(self.block_table), self.seq_lens.ctypes.data, self.batch, self.num_kv_heads,
                      self.head_dim, self.page_size, self.max_pages)


def _chunks(cache: PagedCache, chunk_starts, num_chunks, max_chunks):
    if chunk_starts is None:
        n = (cache.seq_lens + cache.page_size - 1) // cache.page_size
        return None, None, int(max_chunks if max_chunks is not None else cache.max_pages), n.astype(np.int32)
    cs, nc = _i32(chunk_starts), _i32(num_chunks)
    return cs, nc, int(cs.shape[1] - 1), nc


def chunk_meta(cache: PagedCache, chunk_starts=None, num_chunks=None, max_chunks=None):
    """Per-chunk K min / max / mean ([P1] "The comparison" method table).
    Returns (kmin, kmax, cen), each [B][H_kv][max_chunks][D] float64 (NaN past
    a sequence's last chunk)."""
    lib = _load()
    cs, nc, mc, _ = _chunks(cache, chunk_starts, num_chunks, max_chunks)
    shape = (cache.batch, cache.num_kv_heads, mc, cache.head_dim)
    kmin, kmax, cen = (np.full(shape, np.nan) for _ in range(3))
    s = cache._struct()
    lib.orc_chunk_meta(ctypes.byref(s), _p(cs), _p(nc), mc, kmin.ctypes.data, kmax.ctypes.data, cen.ctypes.data)
    return kmin, kmax, cen


def score_decode(q, cache: PagedCache, meta, kind, chunk_starts=None, num_chunks=None, max_chunks=None):
    """Decode chunk scores ([P1] method table; [P3] step 1), GQA group max.
    q [B][H_q][D].  Returns (head_scores [B][H_q][C], scores [B][H_kv][C],
    denom [B][H_kv][C]); entries past a sequence's last chunk are NaN."""
    lib = _load()
    q = to_f64(q)
    cs, nc, mc, _ = _chunks(cache, chunk_starts, num_chunks, max_chunks)
    B, Hq = q.shape[0], q.shape[1]
    hs = np.full((B, Hq, mc), np.nan)
    sc = np.full((B, cache.num_kv_heads, mc), np.nan)
    den = np.full_like(sc, np.nan)
    kmin, kmax, cen = (np.ascontiguousarray(m, dtype=np.float64) for m in meta)
    s = cache._struct()
    lib.orc_score_decode(q.ctypes.data, Hq, ctypes.byref(s), _p(cs), _p(nc), mc, kmin.ctypes.data,
                         kmax.ctypes.data, cen.ctypes.data, int(kind), hs.ctypes.data, sc.ctypes.data,
                         den.ctypes.data)
    return hs, sc, den


def select(scores, n_chunks, mode, *, top_k=0, tokens=0, ratio=0.0, bos=0, eos=0, chunk_len=None, max_sel=None):
    """Per-KV-head selection (fixed top-k [P1]; ratio with forced pages [P2];
    token budget for variable chunks).  scores [B][H_kv][C] (any float dtype,
    widened exactly).  Returns (sel_idx [B][H_kv][max_sel] ascending, -1 padded,
    sel_count [B][H_kv])."""
    lib = _load()
    sc = to_f64(scores)
    B, H, C = sc.shape
    if max_sel is None:
        max_sel = C
    nch = _i32(n_chunks)
    cl = _i32(chunk_len)
    idx = np.full((B, H, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, H), dtype=np.int32)
    rc = lib.orc_select(sc.ctypes.data, B, H, C, nch.ctypes.data, _p(cl), int(mode), int(top_k), int(tokens),
                        float(ratio), int(bos), int(eos), idx.ctypes.data, cnt.ctypes.data, int(max_sel))
    if rc != 0:
        raise ValueError("selection larger than max_sel")
    return idx, cnt


def decode_attn(q, cache: PagedCache, sel_idx=None, sel_count=None, scale=None, chunk_starts=None,
                num_chunks=None, max_chunks=None):
    """Attention of the decode query over the selected chunks only ([P1]
    "attend only to those"); sel_idx None = dense.  Returns [B][H_q][D]."""
    lib = _load()
    q = to_f64(q)
    cs, nc, mc, _ = _chunks(cache, chunk_starts, num_chunks, max_chunks)
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    si, sn = _i32(sel_idx), _i32(sel_count)
    max_sel = 0 if si is None else si.shape[2]
    s = cache._struct()
    lib.orc_decode_attn(q.ctypes.data, Hq, ctypes.byref(s), _p(cs), _p(nc), mc, _p(si), _p(sn), max_sel,
                        float(scale), out.ctypes.data)
    return out


def tile_scores(Q, meta, kind, *, num_kv_heads, tile_rows, block_size, causal=True, tiles=None):
    """Tile score = max over the tile's rows and group heads ([P3] step 2).
    Q [T][H_q][D]; meta = (kmin, kmax, cen) each [H_kv][n_blocks][D] (a leading
    batch axis of 1 is accepted).  Returns (scores, denom) [n_list][H_kv][n_blocks]."""
    lib = _load()
    Q = to_f64(Q)
    T, Hq, D = Q.shape
    kmin, kmax, cen = (np.ascontiguousarray(np.asarray(m, dtype=np.float64).reshape(num_kv_heads, -1, D))
                       for m in meta)
    nb = kmin.shape[1]
    tl = _i32(np.arange((T + tile_rows - 1) // tile_rows) if tiles is None else tiles)
    out = np.zeros((tl.shape[0], num_kv_heads, nb))
    den = np.zeros_like(out)
    lib.orc_tile_scores(Q.ctypes.data, T, Hq, num_kv_heads, D, kmin.ctypes.data, kmax.ctypes.data,
                        cen.ctypes.data, nb, tile_rows, block_size, int(bool(causal)), int(kind), tl.ctypes.data,
                        tl.shape[0], out.ctypes.data, den.ctypes.data)
    return out, den


def quantile(x, p):
    """Empirical quantile, linear interpolation (Hyndman-Fan 7)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    return float(lib.orc_quantile(x.ctypes.data, x.shape[0], float(p)))


def router(tile_scores_, n_visible, k, rho, quantile_p=0.25, fixed_tau=None):
    """Uncertainty router ([P3] "Methodologie" steps 2-5).  tile_scores_
    [n_tiles][H_kv][n_blocks]; n_visible [n_tiles].  Returns a dict with
    kv_idx [n_tiles][H_kv][rho*k], sigma [n_tiles][H_kv], sigma_bar, eligible,
    triggered [n_tiles] and tau."""
    lib = _load()
    ts = to_f64(tile_scores_)
    nt, H, nb = ts.shape
    nv = _i32(n_visible)
    w = rho * k
    kv = np.full((nt, H, w), -1, dtype=np.int32)
    sg = np.zeros((nt, H))
    sb = np.zeros(nt)
    el = np.zeros(nt, dtype=np.uint8)
    tr = np.zeros(nt, dtype=np.uint8)
    tau = ctypes.c_double(0.0)
    lib.orc_router(ts.ctypes.data, nt, H, nb, nv.ctypes.data, int(k), int(rho), float(quantile_p),
                   int(fixed_tau is not None), float(0.0 if fixed_tau is None else fixed_tau), kv.ctypes.data,
                   sg.ctypes.data, sb.ctypes.data, el.ctypes.data, tr.ctypes.data, ctypes.byref(tau))
    return {"kv_idx": kv, "sigma": sg, "sigma_bar": sb, "eligible": el.astype(bool), "triggered": tr.astype(bool),
            "tau": tau.value}


def tile_attn(Q, K, V, *, num_kv_heads, block_size, tile_rows, kv_idx=None, rows=None, scale=None):
    """Causal prefill attention of the listed rows over the blocks of their
    tile's kv_idx entry ([P3] step 5); kv_idx None = dense causal.
    Q [T][H_q][D], K/V [T][H_kv][D].  Returns [n_rows][H_q][D]."""
    lib = _load()
    Q, K, V = to_f64(Q), to_f64(K), to_f64(V)
    T, Hq, D = Q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rl = _i32(np.arange(T) if rows is None else rows)
    kv = _i32(kv_idx)
    stride = 0 if kv is None else kv.shape[-1]
    out = np.zeros((rl.shape[0], Hq, D))
    lib.orc_tile_attn(Q.ctypes.data, K.ctypes.data, V.ctypes.data, T, Hq, num_kv_heads, D, block_size, tile_rows,
                      _p(kv), stride, float(scale), rl.ctypes.data, rl.shape[0], out.ctypes.data)
    return out
