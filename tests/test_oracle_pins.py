"""Pins of the fp64 oracle against things other than itself.

Each test checks one oracle function against a closed form, an invariant the
pages state, a library routine (numpy / scipy), a brute-force enumeration on
tiny inputs, or a worked value under tests/golden/.  They run on the CPU.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from block_sparse_attention_chunk_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c.strip() for c in line.split(";")])
    return rows


def _case(cid=11, lens=(37, 64, 5), hq=6, hkv=2, d=8, page=4, dtype=synth.F32, **kw):
    return synth.make_decode(cid, batch=len(lens), seq_lens=list(lens), num_q_heads=hq, num_kv_heads=hkv,
                             head_dim=d, page_size=page, dtype=dtype, **kw)


def _cache(case):
    return oracle.PagedCache(case.k, case.v, case.block_table, case.seq_lens, case.page_size, case.num_kv_heads,
                             case.head_dim)


def _logical(arr, case, b):
    """Gather sequence b's keys or values into a [L][H][D] array by walking the
    block table page by page (test-side, independent of the oracle)."""
    a = oracle.to_f64(arr)
    L, P = int(case.seq_lens[b]), case.page_size
    out = np.zeros((L, case.num_kv_heads, case.head_dim))
    for t in range(L):
        out[t] = a[case.block_table[b, t // P], :, t % P, :]
    return out


def _intervals(case, b):
    L, P = int(case.seq_lens[b]), case.page_size
    if case.chunk_starts is None:
        return [(s, min(s + P, L)) for s in range(0, L, P)]
    n = int(case.num_chunks[b])
    return [(int(case.chunk_starts[b, c]), int(case.chunk_starts[b, c + 1])) for c in range(n)]


# --------------------------------------------------------------------------
# metadata
# --------------------------------------------------------------------------

@pytest.mark.parametrize("chunked", [False, True])
def test_meta_matches_numpy_reductions(chunked):
    case = _case(lens=(37, 64, 5, 1))
    if chunked:
        starts = [synth.variable_chunks(20 + b, int(L), lo=1, hi=9) for b, L in enumerate(case.seq_lens)]
        synth.with_chunks(case, starts)
    c = _cache(case)
    kmin, kmax, cen = oracle.chunk_meta(c, case.chunk_starts, case.num_chunks)
    for b in range(case.batch):
        K = _logical(case.k, case, b)
        for ci, (s, e) in enumerate(_intervals(case, b)):
            seg = K[s:e]
            np.testing.assert_array_equal(kmin[b, :, ci], seg.min(axis=0))
            np.testing.assert_array_equal(kmax[b, :, ci], seg.max(axis=0))
            np.testing.assert_allclose(cen[b, :, ci], seg.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_meta_one_token_chunks_are_the_key():
    case = _case(lens=(13,))
    synth.with_chunks(case, [np.arange(14)])
    kmin, kmax, cen = oracle.chunk_meta(_cache(case), case.chunk_starts, case.num_chunks)
    K = _logical(case.k, case, 0)
    for t in range(13):
        np.testing.assert_array_equal(kmin[0, :, t], K[t])
        np.testing.assert_array_equal(kmax[0, :, t], K[t])
        np.testing.assert_array_equal(cen[0, :, t], K[t])


def test_meta_token_major_layout():
    # a [T][H][D] cache described by strides must give the same metadata as the
    # same tokens stored page-major
    g = np.random.default_rng(5)
    T, H, D, blk = 40, 3, 4, 8
    K = g.standard_normal((T, H, D))
    c = oracle.PagedCache(K, K, None, [T], blk, H, D, strides=(blk * H * D, D, H * D), max_pages=T // blk)
    kmin, kmax, cen = oracle.chunk_meta(c)
    for bk in range(T // blk):
        seg = K[bk * blk:(bk + 1) * blk]
        np.testing.assert_array_equal(kmin[0, :, bk], seg.min(axis=0))
        np.testing.assert_array_equal(kmax[0, :, bk], seg.max(axis=0))
        np.testing.assert_allclose(cen[0, :, bk], seg.mean(axis=0), rtol=1e-13)


# --------------------------------------------------------------------------
# decode scores
# --------------------------------------------------------------------------

def _scores(case, kind):
    c = _cache(case)
    meta = oracle.chunk_meta(c, case.chunk_starts, case.num_chunks)
    return meta, oracle.score_decode(case.q, c, meta, kind, case.chunk_starts, case.num_chunks)


def test_envelope_is_an_upper_bound_and_group_max():
    # page 1 method table: the envelope is a per-dimension min/max upper bound
    case = _case(lens=(50, 23), hq=8, hkv=2, d=16)
    _, (hs, sc, den) = _scores(case, oracle.ENVELOPE)
    g = case.num_q_heads // case.num_kv_heads
    q = oracle.to_f64(case.q)
    for b in range(case.batch):
        K = _logical(case.k, case, b)
        for ci, (s, e) in enumerate(_intervals(case, b)):
            for j in range(case.num_q_heads):
                true_max = (K[s:e, j // g] @ q[b, j]).max()
                assert hs[b, j, ci] >= true_max - 1e-12 * np.nanmax(den)
            np.testing.assert_array_equal(sc[b, :, ci], hs[b, :, ci].reshape(case.num_kv_heads, g).max(axis=1))


def test_envelope_tight_on_one_token_chunks():
    case = _case(lens=(19,), hq=4, hkv=2, d=16)
    synth.with_chunks(case, [np.arange(20)])
    _, (hs, _, _) = _scores(case, oracle.ENVELOPE)
    K = _logical(case.k, case, 0)
    q = oracle.to_f64(case.q)
    for j in range(4):
        np.testing.assert_allclose(hs[0, j, :19], K[:, j // 2] @ q[0, j], rtol=1e-12, atol=1e-12)


def test_envelope_sign_cases():
    # q >= 0 picks kmax in every dimension, q <= 0 picks kmin
    case = _case(lens=(33,), hq=2, hkv=1, d=8)
    q = oracle.to_f64(case.q)
    q[0, 0] = np.abs(q[0, 0])
    q[0, 1] = -np.abs(q[0, 1])
    case.q = q.astype(np.float32)
    (kmin, kmax, _), (hs, _, _) = _scores(case, oracle.ENVELOPE)
    n = 9
    np.testing.assert_allclose(hs[0, 0, :n], kmax[0, 0, :n] @ q[0, 0], rtol=1e-13)
    np.testing.assert_allclose(hs[0, 1, :n], kmin[0, 0, :n] @ q[0, 1], rtol=1e-13)


def test_centroid_score_is_mean_of_token_dots():
    # linearity: q . mean(k) = mean(q . k)
    case = _case(lens=(45, 16), hq=6, hkv=3, d=12)
    _, (hs, _, _) = _scores(case, oracle.CENTROID)
    q = oracle.to_f64(case.q)
    for b in range(case.batch):
        K = _logical(case.k, case, b)
        for ci, (s, e) in enumerate(_intervals(case, b)):
            for j in range(6):
                ref = (K[s:e, j // 2] @ q[b, j]).mean()
                assert abs(hs[b, j, ci] - ref) <= 1e-12 * (1 + np.abs(K[s:e, j // 2] @ q[b, j]).max())


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def _brute_topk(scores, k, exclude=()):
    """Among all k-subsets (of the non-excluded ids) with maximal score sum,
    the lexicographically smallest: the set a top-k with lower-index tie-break
    must return."""
    ids = [i for i in range(len(scores)) if i not in exclude]
    best, best_set = -np.inf, None
    for comb in itertools.combinations(ids, k):
        s = sum(scores[i] for i in comb)
        if s > best + 0.0 or (s == best and comb < best_set):
            best, best_set = s, comb
    return sorted(best_set)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(4, 10))
    # integer scores (many ties) or continuous scores
    sc = (g.integers(0, 4, size=n) if seed % 2 else g.standard_normal(n)).astype(np.float64)
    for k in range(1, n + 2):
        idx, cnt = oracle.select(sc[None, None], [n], oracle.TOPK, top_k=k)
        want = _brute_topk(list(sc), min(k, n))
        assert cnt[0, 0] == min(k, n)
        assert list(idx[0, 0, :cnt[0, 0]]) == want
        assert np.all(idx[0, 0, cnt[0, 0]:] == -1)


@pytest.mark.parametrize("row", _golden("ratio_budget.txt"))
def test_ratio_budget_counts(row):
    n, ratio, bos, eos, want = int(row[0]), float(row[1]), int(row[2]), int(row[3]), int(row[4])
    sc = np.random.default_rng(n).standard_normal(n)
    idx, cnt = oracle.select(sc[None, None], [n], oracle.RATIO, ratio=ratio, bos=bos, eos=eos)
    assert cnt[0, 0] == want
    sel = set(idx[0, 0, :want].tolist())
    if bos:
        assert 0 in sel
    if eos:
        assert n - 1 in sel


@pytest.mark.parametrize("seed", range(6))
def test_ratio_brute_force(seed):
    g = np.random.default_rng(100 + seed)
    n = int(g.integers(3, 10))
    sc = g.integers(0, 3, size=n).astype(np.float64)
    for bos, eos in [(1, 1), (0, 1), (0, 0)]:
        for ratio in (0.5, 0.375, 0.25):
            idx, cnt = oracle.select(sc[None, None], [n], oracle.RATIO, ratio=ratio, bos=bos, eos=eos)
            K = min(n, max(1 + bos + eos, int(math.floor(n * ratio))))
            forced = sorted(set(([0] if bos else []) + ([n - 1] if eos else [])))
            rest = _brute_topk(list(sc), K - len(forced), exclude=forced)
            assert cnt[0, 0] == K
            assert list(idx[0, 0, :K]) == sorted(forced + rest)


@pytest.mark.parametrize("seed", range(8))
def test_token_budget_prefix_properties(seed):
    g = np.random.default_rng(200 + seed)
    n = int(g.integers(5, 40))
    lens = g.integers(16, 257, size=n).astype(np.int32)
    sc = g.integers(0, 6, size=n).astype(np.float64) if seed % 2 else g.standard_normal(n)
    budget = int(g.integers(16, int(lens.sum()) + 300))
    idx, cnt = oracle.select(sc[None, None], [n], oracle.TOKENS, tokens=budget, chunk_len=lens[None])
    sel = idx[0, 0, :cnt[0, 0]]
    chosen = np.zeros(n, dtype=bool)
    chosen[sel] = True
    rank = sorted(range(n), key=lambda i: (-sc[i], i))
    # (i) fits the budget
    assert lens[chosen].sum() <= budget
    # (ii) a prefix of the score order
    pos = {i: r for r, i in enumerate(rank)}
    if chosen.any() and (~chosen).any():
        assert max(pos[i] for i in np.flatnonzero(chosen)) < min(pos[i] for i in np.flatnonzero(~chosen))
    # (iii) maximal: the next chunk in order would overflow
    if (~chosen).any():
        nxt = min(np.flatnonzero(~chosen), key=lambda i: pos[i])
        assert lens[chosen].sum() + lens[nxt] > budget
    else:
        assert lens.sum() <= budget


@pytest.mark.parametrize("row", _golden("budget_fraction.txt"))
def test_budget_is_page_size_times_topk(row):
    L, P, k, tokens, inv = int(row[0]), int(row[1]), int(row[2]), int(row[3]), float(row[4])
    n = L // P
    sc = np.random.default_rng(k).standard_normal(n)
    idx, cnt = oracle.select(sc[None, None], [n], oracle.TOPK, top_k=k)
    assert cnt[0, 0] * P == tokens == P * k
    assert abs(L / tokens - inv) < 0.35


# --------------------------------------------------------------------------
# decode attention
# --------------------------------------------------------------------------

def _ref_attention(q, K, V, mask=None):
    """Textbook softmax attention with scipy's softmax; masked logits -inf."""
    lg = (K @ q) / math.sqrt(q.shape[0])
    if mask is not None:
        lg = np.where(mask, lg, -np.inf)
    return softmax(lg) @ V


@pytest.mark.parametrize("chunked", [False, True])
def test_decode_dense_and_sparse_match_scipy(chunked):
    case = _case(lens=(41, 9), hq=8, hkv=2, d=8)
    if chunked:
        synth.with_chunks(case, [synth.variable_chunks(30, 41, 2, 11), synth.variable_chunks(31, 9, 2, 5)])
    c = _cache(case)
    _, (_, sc, _) = _scores(case, oracle.ENVELOPE)
    nch = case.n_chunks()
    idx, cnt = oracle.select(np.nan_to_num(sc, nan=-np.inf), nch, oracle.TOPK, top_k=3)
    dense = oracle.decode_attn(case.q, c, chunk_starts=case.chunk_starts, num_chunks=case.num_chunks)
    sparse = oracle.decode_attn(case.q, c, idx, cnt, chunk_starts=case.chunk_starts, num_chunks=case.num_chunks)
    q = oracle.to_f64(case.q)
    g = 4
    for b in range(case.batch):
        K, V = _logical(case.k, case, b), _logical(case.v, case, b)
        iv = _intervals(case, b)
        for j in range(8):
            h = j // g
            np.testing.assert_allclose(dense[b, j], _ref_attention(q[b, j], K[:, h], V[:, h]), rtol=1e-12,
                                       atol=1e-13)
            mask = np.zeros(K.shape[0], dtype=bool)
            for ci in idx[b, h, :cnt[b, h]]:
                s, e = iv[ci]
                mask[s:e] = True
            np.testing.assert_allclose(sparse[b, j], _ref_attention(q[b, j], K[:, h], V[:, h], mask), rtol=1e-12,
                                       atol=1e-13)


def test_full_selection_reproduces_dense_exactly():
    case = _case(lens=(40, 27), hq=4, hkv=2, d=8)
    c = _cache(case)
    n = case.n_chunks()
    _, (_, sc, _) = _scores(case, oracle.CENTROID)
    idx, cnt = oracle.select(np.nan_to_num(sc, nan=-np.inf), n, oracle.TOPK, top_k=1000)
    np.testing.assert_array_equal(oracle.decode_attn(case.q, c, idx, cnt), oracle.decode_attn(case.q, c))


def test_decode_closed_forms():
    case = _case(lens=(30,), hq=2, hkv=1, d=4, page=4)
    k = oracle.to_f64(case.k)
    v = oracle.to_f64(case.v)
    # all keys equal -> uniform weights -> output = mean of the attended values
    k[:] = k[0, 0, 0]
    c = oracle.PagedCache(k, v, case.block_table, case.seq_lens, 4, 1, 4)
    V = _logical(v, case, 0)
    np.testing.assert_allclose(oracle.decode_attn(case.q, c)[0, 1], V[:, 0].mean(axis=0), rtol=1e-13)
    # a single selected one-token chunk -> output = that token's value
    synth.with_chunks(case, [np.arange(31)])
    idx = np.full((1, 1, 30), -1, np.int32)
    idx[0, 0, 0] = 17
    out = oracle.decode_attn(case.q, c, idx, np.array([[1]]), chunk_starts=case.chunk_starts,
                             num_chunks=case.num_chunks)
    np.testing.assert_allclose(out[0, 0], V[17, 0], rtol=1e-15)


def test_decode_invariant_under_block_table_permutation():
    a = _case(cid=40, lens=(35, 20), hq=4, hkv=2, d=8)
    c1 = _cache(a)
    # move every physical page somewhere else and rewrite the table to match
    perm = np.random.default_rng(3).permutation(a.k.shape[0])
    inv = np.argsort(perm)
    k2, v2 = a.k[perm], a.v[perm]
    bt2 = inv[a.block_table].astype(np.int32)
    c2 = oracle.PagedCache(k2, v2, bt2, a.seq_lens, a.page_size, 2, 8)
    np.testing.assert_array_equal(oracle.decode_attn(a.q, c1), oracle.decode_attn(a.q, c2))
    m1 = oracle.chunk_meta(c1)
    m2 = oracle.chunk_meta(c2)
    for x, y in zip(m1, m2):
        np.testing.assert_array_equal(x, y)


# --------------------------------------------------------------------------
# router: sigma, quantile, trigger, expansion
# --------------------------------------------------------------------------

def _router_one(scores, k, rho=2, fixed=None):
    s = np.asarray(scores, dtype=np.float64)
    return oracle.router(s[None, None], [len(s)], k, rho, fixed_tau=fixed)


@pytest.mark.parametrize("row", _golden("sigma_cases.txt"))
def test_sigma_worked_cases(row):
    k = int(row[0])
    sc = [float(x) for x in row[1].split()]
    want = float(row[2])
    r = _router_one(sc, k)
    assert abs(r["sigma"][0, 0] - want) <= 1e-12


def test_sigma_range_and_affine_invariance():
    g = np.random.default_rng(7)
    ts = g.standard_normal((50, 3, 40))
    nv = g.integers(1, 41, size=50)
    r = oracle.router(ts, nv, 8, 2)
    assert np.all((r["sigma"] >= 0) & (r["sigma"] <= 1))
    r2 = oracle.router(ts * 4.0, nv, 8, 2)
    np.testing.assert_array_equal(r["sigma"], r2["sigma"])
    r3 = oracle.router(ts * 3.0 + 11.0, nv, 8, 2)
    np.testing.assert_allclose(r["sigma"], r3["sigma"], atol=1e-12)
    # tiles with at most k visible blocks have no cut-off
    assert np.all(r["sigma"][nv <= 8] == 1.0)
    assert not np.any(r["eligible"][nv <= 8])


@pytest.mark.parametrize("p", [0.0, 0.25, 0.5, 0.9, 1.0])
def test_quantile_matches_numpy(p):
    x = np.random.default_rng(8).standard_normal(37)
    assert abs(oracle.quantile(x, p) - np.quantile(x, p, method="linear")) <= 1e-15 * np.abs(x).max()


@pytest.mark.parametrize("row", _golden("trigger_count.txt"))
def test_trigger_count(row):
    m, p, want = int(row[0]), float(row[1]), int(row[2])
    g = np.random.default_rng(m)
    # one head, m eligible tiles with distinct margins built from three scores
    nb = 3
    ts = np.zeros((m, 1, nb))
    ts[:, 0, 0] = 1.0
    ts[:, 0, 2] = 0.0
    ts[:, 0, 1] = g.permutation(m) / (m + 1.0) + 0.5 / (m + 1.0)   # sigma = ts[...,1], distinct
    r = oracle.router(ts, np.full(m, nb), 2, 2, quantile_p=p)
    # k = 2: sigma = (s_1 - s_2) / (s_0 - s_2) = middle score
    np.testing.assert_allclose(r["sigma"][:, 0], ts[:, 0, 1], rtol=1e-15)
    assert abs(r["tau"] - np.quantile(r["sigma_bar"], p)) <= 1e-15
    assert int(r["triggered"].sum()) == want == math.ceil(p * (m - 1))


def _router_step4_golden():
    tiles, quant = [], []
    for row in _golden("router_step4.txt"):
        if row[0] == "tile":
            tiles.append(dict(visible=int(row[1]), scores=[[float(x) for x in row[2].split()],
                                                           [float(x) for x in row[3].split()]],
                              sigma=[float(row[4]), float(row[5])], mean=float(row[6]), eligible=bool(int(row[7])),
                              kv_idx=[[int(x) for x in row[8].split()], [int(x) for x in row[9].split()]]))
        elif row[0] == "quantile":
            quant.append((float(row[1]), float(row[2]), sorted(int(x) for x in row[3].split())))
    return tiles, quant


@pytest.mark.parametrize("qrow", range(2))
def test_router_head_mean_and_eligible_quantile(qrow):
    """Step 4 of the router on a hand-worked case with two KV heads of
    different margins and ineligible tiles beside eligible ones: the mean over
    heads, the quantile over eligible tiles only, the strict trigger and the
    expansion (tests/golden/router_step4.txt)."""
    tiles, quant = _router_step4_golden()
    p, want_tau, want_trig = quant[qrow]
    ts = np.array([t["scores"] for t in tiles], dtype=np.float64)
    nv = [t["visible"] for t in tiles]
    r = oracle.router(ts, nv, 2, 2, quantile_p=p)
    for i, t in enumerate(tiles):
        np.testing.assert_allclose(r["sigma"][i], t["sigma"], rtol=0, atol=1e-15)
        assert abs(r["sigma_bar"][i] - t["mean"]) <= 1e-15
        assert bool(r["eligible"][i]) == t["eligible"]
    assert abs(r["tau"] - want_tau) <= 1e-15
    assert sorted(np.flatnonzero(r["triggered"]).tolist()) == want_trig
    if p == 0.25:
        for i, t in enumerate(tiles):
            assert r["kv_idx"][i].tolist() == t["kv_idx"]


@pytest.mark.parametrize("seed", range(4))
def test_router_sets_brute_force_and_prefix(seed):
    g = np.random.default_rng(300 + seed)
    nt, H, nb, k, rho = 12, 2, 9, 3, 2
    ts = g.integers(0, 5, size=(nt, H, nb)).astype(np.float64) if seed % 2 else g.standard_normal((nt, H, nb))
    nv = np.minimum(np.arange(nt) + 1, nb)
    lo = oracle.router(ts, nv, k, rho, fixed_tau=-np.inf)     # nothing triggers
    hi = oracle.router(ts, nv, k, rho, fixed_tau=np.inf)      # every eligible tile triggers
    assert not lo["triggered"].any()
    assert np.array_equal(hi["triggered"], hi["eligible"])
    for t in range(nt):
        for h in range(H):
            n = nv[t]
            a = lo["kv_idx"][t, h]
            b = hi["kv_idx"][t, h]
            ka, kb = min(k, n), (min(rho * k, n) if n > k else min(k, n))
            assert list(a[:ka]) == _brute_topk(list(ts[t, h, :n]), ka)
            assert list(b[:kb]) == _brute_topk(list(ts[t, h, :n]), kb)
            assert np.all(a[ka:] == -1) and np.all(b[kb:] == -1)
            assert set(a[:ka]) <= set(b[:kb])
            assert np.all(a[:ka] < n)


# --------------------------------------------------------------------------
# tile scores and tile attention (prefill)
# --------------------------------------------------------------------------

def _prefill(seed=9, T=40, hq=6, hkv=2, d=8):
    g = np.random.default_rng(seed)
    return (g.standard_normal((T, hq, d)), g.standard_normal((T, hkv, d)), g.standard_normal((T, hkv, d)))


def _block_meta(K, blk):
    T, H, D = K.shape
    c = oracle.PagedCache(K, K, None, [T], blk, H, D, strides=(blk * H * D, D, H * D),
                          max_pages=(T + blk - 1) // blk)
    return oracle.chunk_meta(c)


def test_tile_scores_centroid_matches_numpy_and_causality():
    Q, K, _ = _prefill()
    T, blk, g = 40, 8, 3
    meta = _block_meta(K, blk)
    sc, _ = oracle.tile_scores(Q, meta, oracle.CENTROID, num_kv_heads=2, tile_rows=blk, block_size=blk)
    for t in range(T // blk):
        for h in range(2):
            for bk in range(T // blk):
                if bk > t:
                    assert sc[t, h, bk] == -np.inf
                    continue
                rows = Q[t * blk:(t + 1) * blk, h * g:(h + 1) * g]           # [rows][g][D]
                dots = rows @ K[bk * blk:(bk + 1) * blk, h].T              # [rows][g][keys]
                assert abs(sc[t, h, bk] - dots.mean(axis=-1).max()) <= 1e-12 * (1 + np.abs(dots).max())


def test_tile_scores_envelope_bound_and_tightness():
    Q, K, _ = _prefill(seed=10)
    blk, g = 8, 3
    meta = _block_meta(K, blk)
    sc, den = oracle.tile_scores(Q, meta, oracle.ENVELOPE, num_kv_heads=2, tile_rows=blk, block_size=blk)
    for t in range(5):
        for h in range(2):
            for bk in range(t + 1):
                rows = Q[t * blk:(t + 1) * blk, h * g:(h + 1) * g]
                true = (rows @ K[bk * blk:(bk + 1) * blk, h].T).max()
                assert sc[t, h, bk] >= true - 1e-12 * den[t, h, bk]
    # one-key blocks and one-row tiles: the bound is tight
    m1 = _block_meta(K, 1)
    s1, _ = oracle.tile_scores(Q, m1, oracle.ENVELOPE, num_kv_heads=2, tile_rows=1, block_size=1)
    for r in (0, 7, 39):
        for h in range(2):
            for p in range(r + 1):
                true = (Q[r, h * g:(h + 1) * g] @ K[p, h]).max()
                assert abs(s1[r, h, p] - true) <= 1e-12 * (1 + abs(true))


def test_tile_attention_matches_scipy_dense_and_sparse():
    Q, K, V = _prefill(seed=12, T=48)
    blk, g = 8, 3
    rows = np.array([0, 5, 8, 23, 40, 47])
    dense = oracle.tile_attn(Q, K, V, num_kv_heads=2, block_size=blk, tile_rows=blk, rows=rows)
    nt = 6
    kv = np.full((nt, 2, 4), -1, np.int32)
    g2 = np.random.default_rng(1)
    for t in range(nt):
        for h in range(2):
            ch = np.sort(g2.choice(t + 1, size=min(2, t + 1), replace=False))
            kv[t, h, :len(ch)] = ch
    sparse = oracle.tile_attn(Q, K, V, num_kv_heads=2, block_size=blk, tile_rows=blk, kv_idx=kv, rows=rows)
    for ir, r in enumerate(rows):
        t = r // blk
        for j in range(6):
            h = j // g
            causal = np.arange(48) <= r
            np.testing.assert_allclose(dense[ir, j], _ref_attention(Q[r, j], K[:, h], V[:, h], causal), rtol=1e-12,
                                       atol=1e-13)
            sel = np.zeros(48, dtype=bool)
            for bk in kv[t, h]:
                if bk >= 0:
                    sel[bk * blk:(bk + 1) * blk] = True
            np.testing.assert_allclose(sparse[ir, j], _ref_attention(Q[r, j], K[:, h], V[:, h], causal & sel),
                                       rtol=1e-12, atol=1e-13)
    # every visible block selected -> dense causal, bit for bit
    full = np.full((nt, 2, nt), -1, np.int32)
    for t in range(nt):
        full[t, :, :t + 1] = np.arange(t + 1)
    np.testing.assert_array_equal(
        oracle.tile_attn(Q, K, V, num_kv_heads=2, block_size=blk, tile_rows=blk, kv_idx=full, rows=rows), dense)
    # keys after a row never matter
    K2, V2 = K.copy(), V.copy()
    K2[24:] = 100.0
    V2[24:] = -100.0
    early = rows[rows < 24]
    np.testing.assert_array_equal(
        oracle.tile_attn(Q, K2, V2, num_kv_heads=2, block_size=blk, tile_rows=blk, rows=early),
        dense[:len(early)])
