"""GPU-vs-oracle parity of the router prefill path through the C ABI: block
metadata over a token-major cache, query-tile scores (both backbones), the
uncertainty router (sigma, head average, quantile threshold, trigger,
sentinel-padded kv_idx) and causal tile attention, sparse and dense.

Workloads: 28 q / 4 KV heads, d 128, bf16, 64-token blocks and 64-row tiles
with grouped needle blocks and two RMS-normalised KV heads; a 4,096-token
instance (k = 8), a ragged 1,000-token instance, and the full 131,072-token
prefill with k = 32, rho = 2, quantile 0.25 checked on sampled tiles and rows.
"""
import math

import numpy as np
import pytest

import oracle
from block_sparse_attention_chunk_amd import synth
from parity_lib import ATTN_ABS, SCORE_REL, log, max_abs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_chunk_amd import _abi
    _abi.lib()
    return torch.device("cuda:0")


def _np(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def gpu_prefill(pc, dev, kind, k, rho, quantile=0.25, dense=False):
    from block_sparse_attention_chunk_amd import ops
    kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(pc.v, dev),
                     torch.tensor([pc.T], dtype=torch.int32, device=dev), pc.block, token_major=True)
    q = ops.upload(pc.q, dev)
    meta = ops.build_chunk_meta(kv)
    ts = ops.score_chunks(q, kv, meta, kind, rows_per_query=pc.tile, causal=True)
    r = ops.select_topk_router(ts, k=k, rho=rho, quantile=quantile)
    out = ops.sparse_attn_tile_prefill(q, kv, r["kv_idx"])
    dout = ops.sparse_attn_tile_prefill(q, kv, None) if dense else None
    torch.cuda.synchronize()
    res = {"kmin": _np(meta.kmin), "kmax": _np(meta.kmax), "cen": _np(meta.centroid), "ts": _np(ts),
           "kv_idx": _np(r["kv_idx"]), "sigma": _np(r["sigma"]), "sigma_bar": _np(r["sigma_bar"]),
           "triggered": _np(r["triggered"]).astype(bool), "tau": float(_np(r["threshold"])[0])}
    return res, out, dout


def block_meta_oracle(pc):
    T, H, D = pc.k.shape
    c = oracle.PagedCache(pc.k, pc.v, None, [T], pc.block, H, D, strides=(pc.block * H * D, D, H * D),
                          max_pages=(T + pc.block - 1) // pc.block)
    return oracle.chunk_meta(c)


def check_router_on_gpu_scores(g, n_tiles, k, rho):
    """The router's outputs are a function of the tile scores: recompute them
    with the oracle from the GPU's own scores."""
    nv = np.minimum(np.arange(n_tiles) + 1, g["ts"].shape[2])
    ref = oracle.router(g["ts"].astype(np.float64), nv, k, rho)
    assert np.max(np.abs(g["sigma"] - ref["sigma"])) <= 1e-6
    assert np.max(np.abs(g["sigma_bar"] - ref["sigma_bar"])) <= 1e-6
    # the threshold is the quantile of the GPU's own sigma_bar values
    elig = ref["eligible"]
    tau_ref = oracle.quantile(g["sigma_bar"][elig].astype(np.float64), 0.25) if elig.any() else float("nan")
    assert abs(g["tau"] - tau_ref) <= 1e-6
    clear = np.abs(g["sigma_bar"].astype(np.float64) - tau_ref) > 1e-6
    assert np.array_equal(g["triggered"][clear], ref["triggered"][clear])
    same = g["triggered"] == ref["triggered"]
    assert np.array_equal(g["kv_idx"][same], ref["kv_idx"][same])
    m = int(elig.sum())
    return ref, m


def check_router_end_to_end(g, ots, oden, k, rho, quantile=0.25):
    """The GPU pipeline's router against the oracle's own pipeline (oracle
    metadata, oracle tile scores, oracle router).  Each GPU tile score may sit
    up to SCORE_REL * D from the oracle's, and order statistics move no more
    than their inputs, so s_(0), s_(k-1), s_(k) each move by at most
    delta = SCORE_REL * max D over the visible blocks; then
      |sigma' - sigma| <= 4 delta / (s_(0) - s_(k) - 2 delta)  (+1e-6 for fp32),
    sigma_bar moves by at most the mean of its heads' bounds, and the
    threshold, an interpolation of two order statistics of sigma_bar, by at
    most the largest of those.  sigma and tau are gated within these bounds,
    and the trigger set must be exact for every tile whose |sigma_bar - tau|
    exceeds its own bound plus tau's.  Returns (gated tiles, eligible tiles)."""
    n_tiles, H, nb = ots.shape
    nv = np.minimum(np.arange(n_tiles) + 1, nb)
    full = oracle.router(ots, nv, k, rho, quantile_p=quantile)
    eps = np.zeros((n_tiles, H))
    for t in range(n_tiles):
        n = int(nv[t])
        if n <= k:
            continue                              # sigma = 1 on both sides, not eligible
        for h in range(H):
            srt = np.sort(ots[t, h, :n])[::-1]
            delta = SCORE_REL * float(oden[t, h, :n].max())
            gap = srt[0] - srt[k] - 2.0 * delta
            eps[t, h] = 4.0 * delta / gap + 1e-6 if gap > 0 else np.inf
    elig = full["eligible"]
    assert np.array_equal(elig, nv > k)
    fin = np.isfinite(eps)
    assert np.all(np.abs(g["sigma"][fin] - full["sigma"][fin]) <= eps[fin])
    eps_bar = eps.mean(axis=1)
    eps_tau = float(eps_bar[elig].max()) if elig.any() else 0.0
    assert abs(g["tau"] - full["tau"]) <= eps_tau
    clear = np.abs(full["sigma_bar"] - full["tau"]) > eps_bar + eps_tau
    assert np.array_equal(g["triggered"][clear], full["triggered"][clear]), \
        f"trigger differs from the oracle pipeline on tiles {np.flatnonzero(clear & (g['triggered'] != full['triggered']))}"
    return int((clear & elig).sum()), int(elig.sum())


@pytest.mark.parametrize("kind", ["envelope", "centroid"])
def test_router_prefill_small(dev, kind):
    from block_sparse_attention_chunk_amd import ops
    k, rho = 8, 2
    pc = synth.router_prefill(cid=104, T=4096, k=k, groups=8, tied_groups=(1, 3, 5, 7))
    kd = ops.BSA_ENVELOPE if kind == "envelope" else ops.BSA_CENTROID
    log(f"router prefill small {kind}")
    g, out, dout = gpu_prefill(pc, dev, kd, k, rho, dense=True)
    n_tiles = pc.T // pc.tile
    # metadata
    omin, omax, ocen = block_meta_oracle(pc)
    assert np.array_equal(oracle.to_f64(g["kmin"]), omin) and np.array_equal(oracle.to_f64(g["kmax"]), omax)
    assert np.max(np.abs(g["cen"] - ocen)) <= 65 * 2.0 ** -24 * float(np.abs(oracle.to_f64(pc.k)).max())
    # tile scores
    okind = oracle.ENVELOPE if kind == "envelope" else oracle.CENTROID
    ots, oden = oracle.tile_scores(pc.q, (omin, omax, ocen), okind, num_kv_heads=4, tile_rows=64, block_size=64)
    vis = np.isfinite(ots)
    assert np.array_equal(np.isfinite(g["ts"]), vis)
    err = np.abs(g["ts"][vis] - ots[vis]) / oden[vis]
    assert err.max() <= SCORE_REL, err.max()
    # router on the GPU's scores
    ref, m = check_router_on_gpu_scores(g, n_tiles, k, rho)
    assert int(g["triggered"].sum()) == math.ceil(0.25 * (m - 1))
    # sentinels and shape
    for t in range(n_tiles):
        n = min(t + 1, n_tiles)
        keep = min(rho * k if g["triggered"][t] else k, n)
        for h in range(4):
            row = g["kv_idx"][t, h]
            assert np.all(np.diff(row[:keep]) > 0) and np.all(row[keep:] == -1) and np.all(row[:keep] <= t)
    # attention on the GPU's kv_idx, every row
    o = _np(out)
    ref_o = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=4, block_size=64, tile_rows=64, kv_idx=g["kv_idx"])
    e = max_abs(o, ref_o)
    assert e <= ATTN_ABS["bf16"], e
    rows = np.array([0, 1, 63, 64, 1000, 2047, 2048, 4095])
    dref = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=4, block_size=64, tile_rows=64, rows=rows)
    de = max_abs(_np(dout)[rows], dref)
    assert de <= ATTN_ABS["bf16"], de
    # end to end against the oracle's own pipeline, outside the propagated band
    gated, elig = check_router_end_to_end(g, ots, oden, k, rho)
    assert gated >= elig // 2, (gated, elig)
    log(f"  ok: tile score err {err.max():.2e} D, attn err {e:.2e}, dense err {de:.2e}, m={m}, "
        f"trigger set exact against the all-oracle pipeline on {gated} of {elig} eligible tiles")


@pytest.mark.parametrize("quantile,fixed,rho", [(0.0, None, 2), (1.0, None, 2), (0.5, None, 3), (0.25, 0.3, 2),
                                                (0.25, None, 1)])
def test_router_parameters(dev, quantile, fixed, rho):
    """The router's quantile ends (0: nothing triggers, 1: everything below
    the largest sigma_bar does), a fixed threshold instead of the quantile,
    rho = 1 (expansion keeps k) and rho = 3, each recomputed by the oracle from
    the GPU's own tile scores."""
    from block_sparse_attention_chunk_amd import ops
    k = 8
    pc = synth.router_prefill(cid=107, T=4096, k=k, groups=8, tied_groups=(1, 3, 5, 7))
    kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(pc.v, dev),
                     torch.tensor([pc.T], dtype=torch.int32, device=dev), pc.block, token_major=True)
    q = ops.upload(pc.q, dev)
    meta = ops.build_chunk_meta(kv)
    ts = ops.score_chunks(q, kv, meta, ops.BSA_ENVELOPE, rows_per_query=pc.tile, causal=True)
    r = ops.select_topk_router(ts, k=k, rho=rho, quantile=quantile, fixed_threshold=fixed)
    torch.cuda.synchronize()
    g = {"ts": _np(ts), "kv_idx": _np(r["kv_idx"]), "sigma": _np(r["sigma"]), "sigma_bar": _np(r["sigma_bar"]),
         "triggered": _np(r["triggered"]).astype(bool), "tau": float(_np(r["threshold"])[0])}
    n_tiles = pc.T // pc.tile
    nv = np.minimum(np.arange(n_tiles) + 1, g["ts"].shape[2])
    ref = oracle.router(g["ts"].astype(np.float64), nv, k, rho, quantile_p=quantile, fixed_tau=fixed)
    assert np.max(np.abs(g["sigma"] - ref["sigma"])) <= 1e-6
    assert np.max(np.abs(g["sigma_bar"] - ref["sigma_bar"])) <= 1e-6
    elig = ref["eligible"]
    if fixed is None:
        tau_ref = oracle.quantile(g["sigma_bar"][elig].astype(np.float64), quantile)
    else:
        tau_ref = fixed
    assert abs(g["tau"] - tau_ref) <= 1e-6
    clear = np.abs(g["sigma_bar"].astype(np.float64) - tau_ref) > 1e-6
    assert np.array_equal(g["triggered"][clear], ref["triggered"][clear])
    same = g["triggered"] == ref["triggered"]
    assert np.array_equal(g["kv_idx"][same], ref["kv_idx"][same])
    m = int(elig.sum())
    if fixed is None and quantile == 0.0:
        assert not g["triggered"].any()
    if fixed is None and quantile == 1.0:
        assert int(g["triggered"].sum()) >= m - 1 - int(np.sum(g["sigma_bar"][elig] == g["sigma_bar"][elig].max()))
    if rho == 1:
        assert np.all((g["kv_idx"] >= 0).sum(axis=2) == np.minimum(nv, k)[:, None])
    log(f"router q={quantile} fixed={fixed} rho={rho}: {int(g['triggered'].sum())} of {m} eligible tiles triggered")


def test_router_prefill_ragged(dev):
    from block_sparse_attention_chunk_amd import ops
    pc = synth.router_prefill(cid=105, T=1000, num_q_heads=14, num_kv_heads=2, k=4, groups=4, tied_groups=(2,))
    log("router prefill ragged T=1000")
    g, out, dout = gpu_prefill(pc, dev, ops.BSA_ENVELOPE, 4, 2, dense=True)
    n_tiles = (pc.T + 63) // 64
    omin, omax, ocen = block_meta_oracle(pc)
    assert np.array_equal(oracle.to_f64(g["kmax"]), omax)
    ots, oden = oracle.tile_scores(pc.q, (omin, omax, ocen), oracle.ENVELOPE, num_kv_heads=2, tile_rows=64,
                                   block_size=64)
    vis = np.isfinite(ots)
    assert np.array_equal(np.isfinite(g["ts"]), vis)
    assert (np.abs(g["ts"][vis] - ots[vis]) / oden[vis]).max() <= SCORE_REL
    check_router_on_gpu_scores(g, n_tiles, 4, 2)
    check_router_end_to_end(g, ots, oden, 4, 2)
    ref_o = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=2, block_size=64, tile_rows=64, kv_idx=g["kv_idx"])
    assert max_abs(_np(out), ref_o) <= ATTN_ABS["bf16"]
    dref = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=2, block_size=64, tile_rows=64)
    assert max_abs(_np(dout), dref) <= ATTN_ABS["bf16"]


@pytest.mark.parametrize("kind", ["envelope", "centroid"])
def test_router_prefill_16k_end_to_end(dev, kind):
    """16,384 tokens (256 tiles), 28 q / 4 KV heads, k = 32, rho = 2: the
    whole router against the all-oracle pipeline (oracle metadata, every tile
    score, router), gated outside the propagated band, and sampled rows of the
    attention."""
    from block_sparse_attention_chunk_amd import ops
    k, rho = 32, 2
    pc = synth.router_prefill(cid=106, T=16384, k=k, groups=2, tied_groups=(1,))
    kd = ops.BSA_ENVELOPE if kind == "envelope" else ops.BSA_CENTROID
    log(f"router prefill 16K {kind}")
    g, out, _ = gpu_prefill(pc, dev, kd, k, rho)
    omin, omax, ocen = block_meta_oracle(pc)
    assert np.array_equal(oracle.to_f64(g["kmin"]), omin) and np.array_equal(oracle.to_f64(g["kmax"]), omax)
    okind = oracle.ENVELOPE if kind == "envelope" else oracle.CENTROID
    ots, oden = oracle.tile_scores(pc.q, (omin, omax, ocen), okind, num_kv_heads=4, tile_rows=64, block_size=64)
    vis = np.isfinite(ots)
    assert np.array_equal(np.isfinite(g["ts"]), vis)
    err = (np.abs(g["ts"][vis] - ots[vis]) / oden[vis]).max()
    assert err <= SCORE_REL, err
    check_router_on_gpu_scores(g, pc.T // pc.tile, k, rho)
    gated, elig = check_router_end_to_end(g, ots, oden, k, rho)
    assert gated >= elig // 3, (gated, elig)
    rows = np.array([0, 63, 64, 2047, 2048, 5000, 9999, 16383])
    ref_o = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=4, block_size=64, tile_rows=64, kv_idx=g["kv_idx"],
                             rows=rows)
    e = max_abs(_np(out)[rows], ref_o)
    assert e <= ATTN_ABS["bf16"], e
    log(f"  ok: score err {err:.2e} D, trigger set exact on {gated} of {elig} eligible tiles, attn err {e:.2e}")


@pytest.mark.parametrize("kind", ["envelope", "centroid"])
def test_router_prefill_full_size(dev, kind):
    """131,072 tokens, 28 q / 4 KV heads, k = 32, rho = 2, quantile 0.25, both
    scoring backbones: every GPU stage runs at full size; the oracle checks
    sampled blocks, tiles and rows and recomputes the whole router from the
    GPU's tile scores."""
    from block_sparse_attention_chunk_amd import ops
    k, rho = 32, 2
    log(f"router prefill full size ({kind}): generating inputs")
    pc = synth.router_prefill()
    n_tiles = pc.T // pc.tile
    log("  running the GPU pipeline")
    kd = ops.BSA_ENVELOPE if kind == "envelope" else ops.BSA_CENTROID
    okind = oracle.ENVELOPE if kind == "envelope" else oracle.CENTROID
    g, out, _ = gpu_prefill(pc, dev, kd, k, rho)
    o = _np(out)
    del out
    # metadata of sampled blocks
    blocks = np.array([0, 1, 777, 2047])
    T, H, D = pc.k.shape
    kk = oracle.to_f64(pc.k)
    for b in blocks:
        seg = kk[b * 64:(b + 1) * 64]
        assert np.array_equal(oracle.to_f64(g["kmin"])[0, :, b], seg.min(axis=0))
        assert np.array_equal(oracle.to_f64(g["kmax"])[0, :, b], seg.max(axis=0))
        cen_tol = 65 * 2.0 ** -24 * float(np.abs(seg).max())
        assert np.max(np.abs(g["cen"][0, :, b] - seg.mean(axis=0))) <= cen_tol
    # tile scores of sampled tiles
    tiles = np.array([0, 31, 32, 33, 400, 1024, 2047])
    log("  oracle tile scores on sampled tiles")
    meta = (oracle.to_f64(g["kmin"]), oracle.to_f64(g["kmax"]), g["cen"].astype(np.float64))
    ots, oden = oracle.tile_scores(pc.q, meta, okind, num_kv_heads=4, tile_rows=64, block_size=64,
                                   tiles=tiles)
    for i, t in enumerate(tiles):
        vis = np.isfinite(ots[i])
        assert np.array_equal(np.isfinite(g["ts"][t]), vis)
        assert (np.abs(g["ts"][t][vis] - ots[i][vis]) / oden[i][vis]).max() <= SCORE_REL
    log("  oracle router on the GPU's tile scores")
    ref, m = check_router_on_gpu_scores(g, n_tiles, k, rho)
    assert m == 2016
    distinct = len(np.unique(g["sigma_bar"][ref["eligible"]])) == m
    if distinct:
        assert int(g["triggered"].sum()) == 504
    # attention on sampled rows
    rows = np.concatenate([np.arange(0, 64, 9), [64, 2047, 2048 + 5, 65535, 100000, 131071],
                           np.random.default_rng(0).integers(0, T, 8)])
    log(f"  oracle tile attention on {len(rows)} rows")
    ref_o = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=4, block_size=64, tile_rows=64, kv_idx=g["kv_idx"],
                             rows=rows)
    e = max_abs(o[rows], ref_o)
    assert e <= ATTN_ABS["bf16"], e
    near = float(np.mean(g["sigma"][32:] < 0.05))
    log(f"  ok: m={m}, triggered={int(g['triggered'].sum())}, tau={g['tau']:.4f}, sparse attn err {e:.2e}, "
        f"fraction of (tile, head) with sigma < 0.05: {near:.3f}")


@pytest.mark.parametrize("nt,H,nb,causal,k,rho,ties", [
    (300, 3, 300, True, 100, 2, False),     # 200-entry rows, causal
    (40, 2, 3000, False, 85, 3, False),     # 255-entry rows, 256-thread selection (> 2048 blocks)
    (20, 1, 5000, False, 20, 2, False),     # 1024-thread selection (> 4096 blocks)
    (64, 4, 64, True, 8, 2, True),          # integer scores: ties at every cut
    (9, 1, 10, True, 4, 2, False),          # fewer tiles than a workgroup's share
    (33, 2, 300, False, 255, 1, False),     # rho = 1 with k + 1 = 256 sorted scores
    # causal rows of every length, crossing each boundary of the candidate
    # slots per thread (a quarter, half, three quarters or all of the
    # workgroup's share) and of the quantile's slots (m <= 2048, 4096, more)
    (1600, 2, 1600, True, 16, 2, False),    # 128-thread selection: 512 / 1024 / 1536 blocks
    (2200, 1, 2200, True, 20, 2, False),    # 256-thread selection: 1024 / 2048 blocks
    (5000, 1, 5000, True, 20, 2, False),    # 1024-thread selection: 2048 / 4096 blocks; m > 4096
    (7000, 1, 7000, True, 20, 2, False),    # 1024-thread selection: 6144 blocks and past it
])
def test_router_on_synthetic_scores(dev, nt, H, nb, causal, k, rho, ties):
    """The router alone on seeded tile scores, exactly against the oracle
    router on the same scores: sigma, sigma_bar, threshold, trigger set and
    the expanded, sentinel-padded kv_idx rows."""
    from block_sparse_attention_chunk_amd import ops
    g = np.random.default_rng(nt * 7 + k)
    ts = (g.integers(0, 6, size=(nt, H, nb)) if ties else g.standard_normal((nt, H, nb))).astype(np.float32)
    log(f"router on synthetic scores nt={nt} H={H} nb={nb} causal={causal} k={k} rho={rho} ties={ties}")
    r = ops.select_topk_router(torch.tensor(ts, device=dev), k=k, rho=rho, causal=causal)
    torch.cuda.synchronize()
    nv = np.minimum(np.arange(nt) + 1, nb) if causal else np.full(nt, nb)
    ref = oracle.router(ts.astype(np.float64), nv, k, rho)
    sg, sb = _np(r["sigma"]), _np(r["sigma_bar"])
    assert np.max(np.abs(sg - ref["sigma"])) <= 1e-6
    assert np.max(np.abs(sb - ref["sigma_bar"])) <= 1e-6
    elig = ref["eligible"]
    tau = float(_np(r["threshold"])[0])
    tau_ref = oracle.quantile(sb[elig].astype(np.float64), 0.25) if elig.any() else float("nan")
    assert (np.isnan(tau) and np.isnan(tau_ref)) or abs(tau - tau_ref) <= 1e-6
    trig = _np(r["triggered"]).astype(bool)
    ref2 = oracle.router(ts.astype(np.float64), nv, k, rho, fixed_tau=tau_ref)   # oracle trigger at the GPU's values
    clear = np.abs(sb.astype(np.float64) - tau_ref) > 1e-6
    assert np.array_equal(trig[clear], ref2["triggered"][clear])
    kv = _np(r["kv_idx"])
    same = trig == ref["triggered"]
    assert np.array_equal(kv[same], ref["kv_idx"][same])
    for t in np.flatnonzero(~same):          # a trigger decided within 1e-6 of the threshold: still a valid row
        for h in range(H):
            keep = min(rho * k if trig[t] else k, nv[t])
            row = kv[t, h]
            assert np.all(np.diff(row[:keep]) > 0) and np.all(row[keep:] == -1)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_tile_attention_group_sizes(dev, g):
    """Tile attention for every supported GQA group size on a ragged
    777-token prefill, over random ascending block lists (sentinel padded)
    and dense causal; every row against the oracle."""
    from block_sparse_attention_chunk_amd import ops
    pc = synth.router_prefill(cid=110 + g, T=777, num_q_heads=2 * g, num_kv_heads=2, k=3, groups=4,
                              tied_groups=(1,))
    log(f"tile attention g={g}")
    n_tiles = (pc.T + 63) // 64
    rng = np.random.default_rng(g)
    stride = 6
    kv_idx = np.full((n_tiles, 2, stride), -1, np.int32)
    for t in range(n_tiles):
        for h in range(2):
            n = int(rng.integers(1, min(t + 1, stride) + 1))
            blocks = np.sort(rng.choice(t + 1, size=n, replace=False))
            if t > 0 and rng.random() < 0.5:
                blocks[-1] = t if t not in blocks[:-1] else blocks[-1]   # often include the diagonal
                blocks = np.unique(blocks)
            kv_idx[t, h, :len(blocks)] = blocks
    kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(pc.v, dev),
                     torch.tensor([pc.T], dtype=torch.int32, device=dev), pc.block, token_major=True)
    q = ops.upload(pc.q, dev)
    out = ops.sparse_attn_tile_prefill(q, kv, torch.tensor(kv_idx, device=dev))
    dout = ops.sparse_attn_tile_prefill(q, kv, None)
    torch.cuda.synchronize()
    ref = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=2, block_size=64, tile_rows=64, kv_idx=kv_idx)
    e = max_abs(_np(out), ref)
    assert e <= ATTN_ABS["bf16"], e
    dref = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=2, block_size=64, tile_rows=64)
    de = max_abs(_np(dout), dref)
    assert de <= ATTN_ABS["bf16"], de
    log(f"  ok: sparse err {e:.2e}, dense err {de:.2e}")


@pytest.mark.parametrize("g", [1, 3, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_tile_scores_group_sizes(dev, g, causal):
    """Tile scores (both backbones) for several GQA group sizes -- different
    copy shares per wave in the staged pipeline -- causal and not, on a
    ragged 1,500-token prefill (24 tiles, more than one 16-block group)."""
    from block_sparse_attention_chunk_amd import ops
    pc = synth.router_prefill(cid=120 + g, T=1500, num_q_heads=2 * g, num_kv_heads=2, k=3, groups=4,
                              tied_groups=(1,))
    kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(pc.v, dev),
                     torch.tensor([pc.T], dtype=torch.int32, device=dev), pc.block, token_major=True)
    q = ops.upload(pc.q, dev)
    meta = ops.build_chunk_meta(kv)
    omin, omax, ocen = block_meta_oracle(pc)
    for kind, okind in ((ops.BSA_ENVELOPE, oracle.ENVELOPE), (ops.BSA_CENTROID, oracle.CENTROID)):
        log(f"tile scores g={g} causal={causal} kind={kind}")
        ts = _np(ops.score_chunks(q, kv, meta, kind, rows_per_query=64, causal=causal))
        ots, oden = oracle.tile_scores(pc.q, (omin, omax, ocen), okind, num_kv_heads=2, tile_rows=64,
                                       block_size=64, causal=causal)
        vis = np.isfinite(ots)
        assert np.array_equal(np.isfinite(ts), vis)
        err = np.abs(ts[vis] - ots[vis]) / oden[vis]
        assert err.max() <= SCORE_REL, err.max()


def test_tile_attention_value_beyond_fp16_range_is_not_silent(dev):
    """P.V runs in fp16, so a finite bf16 value beyond the fp16 range
    (|v| > 65504) cannot be represented.  It is not dropped silently: every
    row whose selected blocks contain it comes out non-finite (in the
    value's KV head), and every other row stays finite and matches the
    oracle."""
    from block_sparse_attention_chunk_amd import ops
    pc = synth.router_prefill(cid=131, T=640, num_q_heads=4, num_kv_heads=2, k=2, groups=4, tied_groups=(1,))
    v = pc.v.copy()
    tok, head = 200, 1                     # block 3, KV head 1
    v[tok, head, 5] = 0x47c3               # bf16 bits of 99840.0: finite in bf16, beyond fp16
    n_tiles = (pc.T + 63) // 64
    kv_idx = np.full((n_tiles, 2, 2), -1, np.int32)
    for t in range(n_tiles):
        kv_idx[t, 0, :2 if t > 0 else 1] = [0, t] if t > 0 else [0]          # head 0: first and diagonal block
        kv_idx[t, 1, :2 if t > 0 else 1] = [0, 1] if t > 0 else [0]          # head 1 avoids block 3 ...
    kv_idx[6, 1, :2] = [3, 6]              # ... except tile 6, which attends to the block holding the value
    log("tile attention with a value beyond the fp16 range")
    kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(v, dev), torch.tensor([pc.T], dtype=torch.int32, device=dev),
                     pc.block, token_major=True)
    out = _np(ops.sparse_attn_tile_prefill(ops.upload(pc.q, dev), kv, torch.tensor(kv_idx, device=dev)))
    torch.cuda.synchronize()
    g = pc.num_q_heads // pc.num_kv_heads
    bad_rows = np.arange(6 * 64, 7 * 64)
    bad_heads = np.arange(head * g, (head + 1) * g)
    assert not np.all(np.isfinite(out[np.ix_(bad_rows, bad_heads)]))
    mask = np.ones(out.shape, bool)
    mask[np.ix_(bad_rows, bad_heads)] = False
    assert np.all(np.isfinite(out[mask]))
    ref = oracle.tile_attn(pc.q, pc.k, v, num_kv_heads=2, block_size=64, tile_rows=64, kv_idx=kv_idx)
    assert np.max(np.abs(out[mask] - ref[mask])) <= ATTN_ABS["bf16"]


def test_tile_attention_empty_and_short_block_lists(dev):
    """Rows with nothing to attend to: a tile whose kv_idx row holds no
    block (all -1) comes out NaN, the softmax over an empty set, exactly
    where the oracle's does; a row cut short by an entry past the diagonal
    ends there; every other row matches the oracle."""
    from block_sparse_attention_chunk_amd import ops
    pc = synth.router_prefill(cid=3, T=200, num_q_heads=4, num_kv_heads=2, k=2, groups=2, tied_groups=(),
                              rms_heads=())
    n_tiles = (pc.T + 63) // 64
    kv_idx = np.full((n_tiles, 2, 3), -1, np.int32)
    kv_idx[1, 0, :2] = [0, 1]
    kv_idx[2, 1, 0] = 2
    kv_idx[3, 0, :3] = [1, 3, 4]           # block 4 lies past tile 3: the list ends before it
    kv_idx[3, 1, :1] = [0]
    log("tile attention with empty and short block lists")
    kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(pc.v, dev),
                     torch.tensor([pc.T], dtype=torch.int32, device=dev), pc.block, token_major=True)
    out = _np(ops.sparse_attn_tile_prefill(ops.upload(pc.q, dev), kv, torch.tensor(kv_idx, device=dev)))
    torch.cuda.synchronize()
    ref = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=2, block_size=64, tile_rows=64, kv_idx=kv_idx)
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    assert np.isnan(out[0:64]).all() and np.isnan(out[64:128, 2:4]).all()
    fin = ~np.isnan(ref)
    assert fin.sum() > 0 and np.max(np.abs(out[fin] - ref[fin])) <= ATTN_ABS["bf16"]


def _random_prefill_config(i):
    """The i-th seeded router-prefill configuration: length (ragged), KV
    heads, group size, k, rho, quantile and scoring drawn together."""
    r = np.random.default_rng(7000 + i)
    return dict(T=int(r.integers(65, 5000)), hkv=int(r.choice([1, 2, 4])), g=int(r.integers(1, 9)),
                k=int(r.integers(1, 13)), rho=int(r.choice([1, 2, 3])), quantile=float(r.choice([0.1, 0.25, 0.5, 0.9])),
                kind=str(r.choice(["envelope", "centroid"])))


@pytest.mark.parametrize("i", range(10))
def test_randomized_prefill_configurations(dev, i):
    """Seeded random router prefills through the whole pipeline against the
    oracle: block metadata, tile scores, the router on the GPU's scores
    (exact away from the threshold) and against the oracle's own pipeline
    (within the propagated score bound), and sparse and dense tile attention
    on every row."""
    from block_sparse_attention_chunk_amd import ops
    c = _random_prefill_config(i)
    k, rho, qp = c["k"], c["rho"], c["quantile"]
    log(f"random prefill {i}: {c}")
    pc = synth.router_prefill(cid=7100 + i, T=c["T"], num_q_heads=c["hkv"] * c["g"], num_kv_heads=c["hkv"], k=k,
                              groups=4, tied_groups=(1, 3), rms_heads=(0,))
    kd = ops.BSA_ENVELOPE if c["kind"] == "envelope" else ops.BSA_CENTROID
    g, out, dout = gpu_prefill(pc, dev, kd, k, rho, quantile=qp, dense=True)
    n_tiles = (pc.T + 63) // 64
    omin, omax, ocen = block_meta_oracle(pc)
    assert np.array_equal(oracle.to_f64(g["kmin"]), omin) and np.array_equal(oracle.to_f64(g["kmax"]), omax)
    assert np.max(np.abs(g["cen"] - ocen)) <= 65 * 2.0 ** -24 * float(np.abs(oracle.to_f64(pc.k)).max())
    okind = oracle.ENVELOPE if c["kind"] == "envelope" else oracle.CENTROID
    ots, oden = oracle.tile_scores(pc.q, (omin, omax, ocen), okind, num_kv_heads=c["hkv"], tile_rows=64,
                                   block_size=64)
    vis = np.isfinite(ots)
    assert np.array_equal(np.isfinite(g["ts"]), vis)
    assert (np.abs(g["ts"][vis] - ots[vis]) / oden[vis]).max() <= SCORE_REL
    # the router on the GPU's own scores
    nv = np.minimum(np.arange(n_tiles) + 1, g["ts"].shape[2])
    ref = oracle.router(g["ts"].astype(np.float64), nv, k, rho, quantile_p=qp)
    assert np.max(np.abs(g["sigma"] - ref["sigma"])) <= 1e-6
    assert np.max(np.abs(g["sigma_bar"] - ref["sigma_bar"])) <= 1e-6
    elig = ref["eligible"]
    if elig.any():
        tau_ref = oracle.quantile(g["sigma_bar"][elig].astype(np.float64), qp)
        assert abs(g["tau"] - tau_ref) <= 1e-6
        ref2 = oracle.router(g["ts"].astype(np.float64), nv, k, rho, fixed_tau=tau_ref)
        clear = np.abs(g["sigma_bar"].astype(np.float64) - tau_ref) > 1e-6
        assert np.array_equal(g["triggered"][clear], ref2["triggered"][clear])
        check_router_end_to_end(g, ots, oden, k, rho, qp)
    else:                                    # no tile has a cut-off: nothing triggers
        assert np.isnan(g["tau"]) and not g["triggered"].any()
    same = g["triggered"] == ref["triggered"]
    assert np.array_equal(g["kv_idx"][same], ref["kv_idx"][same])
    # attention on the GPU's kv_idx, every row; dense causal
    o = _np(out)
    ref_o = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=c["hkv"], block_size=64, tile_rows=64,
                             kv_idx=g["kv_idx"])
    assert max_abs(o, ref_o) <= ATTN_ABS["bf16"]
    dref = oracle.tile_attn(pc.q, pc.k, pc.v, num_kv_heads=c["hkv"], block_size=64, tile_rows=64)
    assert max_abs(_np(dout), dref) <= ATTN_ABS["bf16"]
