"""GPU-vs-oracle parity of the decode path (metadata, scores, selection,
split-K attention, dense baseline, fused selection + attention) through the
C ABI.

Workloads: the tiny fp32 decode; the 32:4-head, d 128 replay-shaped decode at
29,504 tokens (budgets 4096 / 8192, envelope and centroid); the same with
variable 16-256-token chunks (token budgets 4096 / 8192 / 16384 plus full
context, and a 16,384-token instance whose 16,384 budget is dense); batched
64:8-head decode with ragged lengths and the seven ratio budgets; the
benchmark's 32,768-token decode records at full size (one sequence, 16
sequences, 64:8 heads at ratio 1/8); NaN in the unused tail slots of partial
pages; several split counts.
"""
import math

import numpy as np
import pytest

import oracle
from block_sparse_attention_chunk_amd import synth
from parity_lib import (ATTN_ABS, check_band, check_scores, gpu_kv, log, max_abs, oracle_cache, oracle_select,
                        unequal_rows_case)

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


def run_decode_case(case, dev, kind, budget, forced=(), splits=(0,), check_dense=True, band_exact_count=True):
    from block_sparse_attention_chunk_amd import ops
    log(f"case {case.name} kind={kind} budget={budget}")
    kv, chunks = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    meta = ops.build_chunk_meta(kv, chunks)
    scores = ops.score_chunks(q, kv, meta, kind, chunks=chunks)
    sel, cnt = ops.select_topk(scores, kv, budget, chunks)
    outs = {s: ops.sparse_attn_decode(q, kv, sel, cnt, chunks, num_splits=s) for s in splits}
    dense = ops.sparse_attn_decode(q, kv, None, None, chunks) if check_dense else None
    # the fused selection + attention (16-token pages): same kept set, and the
    # same output bits as the two calls with the same num_splits (with 0 on a
    # large batch both take the balanced schedule), and, with the split grid
    # named explicitly, as the two calls on that grid
    fused = {}
    if chunks is None and case.page_size == 16:
        for s in splits:
            fsel, fcnt = torch.full_like(sel, -7), torch.full_like(cnt, -7)
            fout = ops.select_attn_decode(q, kv, scores, budget, num_splits=s, sel_idx=fsel, sel_count=fcnt)
            grid = ops.decode_num_splits(kv, case.num_q_heads, budget.max_selected(kv.max_pages), s)
            gout = ops.select_attn_decode(q, kv, scores, budget, num_splits=grid)
            fused[s] = (fout, fsel, fcnt, gout, ops.sparse_attn_decode(q, kv, sel, cnt, num_splits=grid))
    torch.cuda.synchronize()
    for s, (fout, fsel, fcnt, gout, sout) in fused.items():
        assert torch.equal(fsel, sel) and torch.equal(fcnt, cnt), f"fused selection differs (splits={s})"
        assert torch.equal(fout, outs[s]), f"fused output not bit-identical (splits={s})"
        assert torch.equal(gout, sout), f"fused output not bit-identical on the split grid (splits={s})"
    kmin, kmax, cen = _np(meta.kmin), _np(meta.kmax), _np(meta.centroid)
    scores, sel, cnt = _np(scores), _np(sel), _np(cnt)

    oc = oracle_cache(case)
    omin, omax, ocen = oracle.chunk_meta(oc, case.chunk_starts, case.num_chunks)
    n = case.n_chunks()
    wide = oracle.to_f64
    # 1. metadata: min / max bit-exact, centroid within the fp32 summation bound
    kabs = float(np.nanmax(np.abs(wide(case.k))))
    nmax = int(np.max(np.diff(case.chunk_starts, axis=1))) if case.chunk_starts is not None else case.page_size
    cen_tol = (nmax + 1) * 2.0 ** -24 * kabs
    for b in range(case.batch):
        nb = int(n[b])
        assert np.array_equal(wide(kmin)[b, :, :nb], omin[b, :, :nb]), "kmin not bit-exact"
        assert np.array_equal(wide(kmax)[b, :, :nb], omax[b, :, :nb]), "kmax not bit-exact"
        assert np.max(np.abs(cen[b, :, :nb] - ocen[b, :, :nb])) <= cen_tol
    # 2. scores within 1e-4 D
    _, osc, oden = oracle.score_decode(case.q, oc, (omin, omax, ocen), kind, case.chunk_starts, case.num_chunks)
    worst = check_scores(scores, osc, oden, n, case.name)
    # 3a. selection is an exact function of the scores it is given
    rsel, rcnt = oracle_select(scores.astype(np.float64), case, budget)
    assert np.array_equal(cnt, rcnt), "selection count differs from the oracle on identical scores"
    for b in range(case.batch):
        for h in range(case.num_kv_heads):
            assert np.array_equal(sel[b, h, :cnt[b, h]], rsel[b, h, :rcnt[b, h]]), (b, h)
            assert np.all(sel[b, h, cnt[b, h]:] == -1)
    # 3b. against the oracle's own scores: band rule
    osel, ocnt = oracle_select(osc, case, budget)
    diffs = check_band(sel, cnt, osel, ocnt, osc, oden, n, forced, exact_count=band_exact_count)
    # 4. attention on the GPU's selection
    ref = oracle.decode_attn(case.q, oc, sel, cnt, chunk_starts=case.chunk_starts, num_chunks=case.num_chunks)
    tol = ATTN_ABS[case.dtype]
    for s, out in outs.items():
        err = max_abs(_np(out), ref)
        assert err <= tol, f"splits={s}: attention max-abs {err:.3g} > {tol}"
    if check_dense:
        dref = oracle.decode_attn(case.q, oc, chunk_starts=case.chunk_starts, num_chunks=case.num_chunks)
        derr = max_abs(_np(dense), dref)
        assert derr <= tol, f"dense max-abs {derr:.3g}"
    log(f"  ok: worst score err {worst:.2e} D, in-band selection diffs {diffs}, attn err "
        f"{max(max_abs(_np(o), ref) for o in outs.values()):.2e}, fused checked: {bool(fused)}")
    return {"sel": sel, "cnt": cnt, "out": _np(next(iter(outs.values()))), "ref": ref, "osel": osel, "ocnt": ocnt}


def test_tiny_fp32_decode(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.tiny_decode()
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.topk(8), splits=(0, 1, 3, 8))
    assert np.all(r["cnt"] == 8)


@pytest.mark.parametrize("kind", ["envelope", "centroid"])
@pytest.mark.parametrize("k", [256, 512])
def test_replay_decode(dev, kind, k):
    from block_sparse_attention_chunk_amd import ops
    case = synth.replay_decode()
    kd = ops.BSA_ENVELOPE if kind == "envelope" else ops.BSA_CENTROID
    r = run_decode_case(case, dev, kd, ops.Budget.topk(k), splits=(0, 1, 7))
    assert np.all(r["cnt"] == k)
    # the planted needle pages are found
    needles = set(case.info["needle_pages"].tolist())
    for h in range(case.num_kv_heads):
        assert needles <= set(r["sel"][0, h, :k].tolist())


@pytest.mark.parametrize("tokens", [4096, 8192, 16384, 1 << 20])
def test_varchunk_decode(dev, tokens):
    from block_sparse_attention_chunk_amd import ops
    case = synth.varchunk_decode()
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.token_budget(tokens), band_exact_count=False,
                        check_dense=tokens == 4096)
    lens = case.chunk_len[0]
    for h in range(case.num_kv_heads):
        tot = int(lens[r["sel"][0, h, :r["cnt"][0, h]]].sum())
        assert tot <= tokens and (tot > tokens - 256 or tot == int(case.seq_lens[0]))
    if tokens >= int(case.seq_lens[0]):
        dense = oracle.decode_attn(case.q, oracle_cache(case), chunk_starts=case.chunk_starts,
                                   num_chunks=case.num_chunks)
        assert max_abs(r["out"], dense) <= ATTN_ABS["bf16"]


def test_varchunk_16k_budget_is_dense(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.varchunk_decode(cid=2, seq_len=16384)
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.token_budget(16384), band_exact_count=False,
                        check_dense=False)
    assert np.all(r["cnt"][0] == case.num_chunks[0])
    dense = oracle.decode_attn(case.q, oracle_cache(case), chunk_starts=case.chunk_starts, num_chunks=case.num_chunks)
    assert max_abs(r["out"], dense) <= ATTN_ABS["bf16"]


@pytest.mark.parametrize("ratio", synth.RATIOS)
@pytest.mark.parametrize("kind", ["centroid", "envelope"])
def test_batched_ratio_small(dev, ratio, kind):
    from block_sparse_attention_chunk_amd import ops
    case = synth.batched_decode(cid=13, batch=5, lo=700, hi=3000)
    bos = 1 if kind == "centroid" else 0
    kd = ops.BSA_CENTROID if kind == "centroid" else ops.BSA_ENVELOPE
    forced = (("bos",) if bos else ()) + ("eos",)
    r = run_decode_case(case, dev, kd, ops.Budget.ratio_budget(ratio, bos, 1), forced=forced,
                        check_dense=ratio == 0.5)
    n = case.n_chunks()
    for b in range(case.batch):
        K = min(int(n[b]), max(2 + bos, int(math.floor(int(n[b]) * ratio))))
        for h in range(case.num_kv_heads):
            s = r["sel"][b, h, :r["cnt"][b, h]]
            assert r["cnt"][b, h] == K
            assert int(n[b]) - 1 in s and (not bos or 0 in s)


def test_nan_tail_slots_are_never_read(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(21, batch=3, seq_lens=[33, 250, 1001], num_q_heads=16, num_kv_heads=2, head_dim=128,
                             pad_value=float("nan"), name="nan-tail")
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.topk(5), splits=(0, 1, 2))
    assert np.all(np.isfinite(r["out"]))


@pytest.mark.parametrize("g", [1, 3, 12, 16])
def test_group_sizes_and_head_dim_64(dev, g):
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(30 + g, batch=2, seq_lens=[517, 1200], num_q_heads=2 * g, num_kv_heads=2, head_dim=64,
                             name=f"g{g}-d64")
    run_decode_case(case, dev, ops.BSA_CENTROID, ops.Budget.topk(12), splits=(0, 1, 5))


def test_page_size_32_uses_general_path(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(40, batch=2, seq_lens=[300, 1000], num_q_heads=8, num_kv_heads=2, head_dim=128,
                             page_size=32, name="page32")
    run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.topk(6), splits=(0, 3))


@pytest.mark.parametrize("page", [8, 32, 64, 256])
def test_other_page_sizes_never_read_past_a_chunk(dev, page):
    """Fixed pages other than 16 tokens (8: the per-token kernel; 32 and 64:
    the 16-token-segment kernel), NaN in every unused tail slot."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(41 + page, batch=3, seq_lens=[37, 300, 1001], num_q_heads=8, num_kv_heads=2,
                             head_dim=128, page_size=page, pad_value=float("nan"), name=f"page{page}-nan")
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.topk(4), splits=(0, 1, 3))
    assert np.all(np.isfinite(r["out"]))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64)])
def test_variable_chunks_other_dtypes_and_head_dims(dev, dtype, d):
    """The segment kernel's float32 path and its head_dim-64 operands: variable
    chunks over a ragged batch, token budget, several split counts."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(60 + d, batch=2, seq_lens=[700, 1900], num_q_heads=8, num_kv_heads=2, head_dim=d,
                             dtype=synth.F32 if dtype == "f32" else synth.BF16, name=f"varchunk-{dtype}-d{d}")
    case = synth.with_chunks(case, [synth.variable_chunks(61, 700, 16, 96), synth.variable_chunks(62, 1900, 16, 96)])
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.token_budget(400), band_exact_count=False,
                        splits=(0, 1, 3))
    lens = case.chunk_len
    for b in range(case.batch):
        for h in range(case.num_kv_heads):
            assert int(lens[b][r["sel"][b, h, :r["cnt"][b, h]]].sum()) <= 400


@pytest.mark.parametrize("layout", ["2048 chunks", "over 2048 chunks"])
def test_long_chunk_lists(dev, layout):
    """Rows of exactly 2048 chunks of 10 tokens (the segment kernel at its
    capacity) and of more than 2048 chunks of 4-12 tokens (the selected and the
    dense call take the per-token kernel instead)."""
    from block_sparse_attention_chunk_amd import ops
    if layout == "2048 chunks":
        case = synth.with_chunks(synth.replay_decode(cid=6, seq_len=20480), [np.arange(0, 20481, 10)])
        assert int(case.num_chunks[0]) == 2048
    else:
        case = synth.with_chunks(synth.replay_decode(cid=5, seq_len=20000), [synth.variable_chunks(5, 20000, 4, 12)])
        assert int(case.num_chunks[0]) > 2048
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.token_budget(12000), band_exact_count=False,
                        splits=(0, 5))
    lens = case.chunk_len[0]
    for h in range(case.num_kv_heads):
        assert int(lens[r["sel"][0, h, :r["cnt"][0, h]]].sum()) <= 12000


def test_deterministic_bits(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.batched_decode(cid=14, batch=4, lo=2000, hi=5000)
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    outs = []
    for _ in range(2):
        meta = ops.build_chunk_meta(kv)
        sc = ops.score_chunks(q, kv, meta, ops.BSA_ENVELOPE)
        sel, cnt = ops.select_topk(sc, kv, ops.Budget.ratio_budget(0.125, 0, 1))
        outs.append(ops.sparse_attn_decode(q, kv, sel, cnt).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("kind,ratio", [("centroid", 0.5), ("centroid", 0.125), ("envelope", 0.5),
                                        ("envelope", 0.0625)])
def test_batched_ratio_full_size(dev, kind, ratio):
    """16 sequences with lengths in [8192, 32768], 64 q / 8 KV heads (the
    benchmark's batched workload): centroid scoring with bos + eos forced,
    envelope scoring with eos only (bos = 0), at the largest ratio and a
    small one; kept counts follow the ratio formula."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.batched_decode()
    bos = 1 if kind == "centroid" else 0
    kd = ops.BSA_CENTROID if kind == "centroid" else ops.BSA_ENVELOPE
    forced = (("bos",) if bos else ()) + ("eos",)
    r = run_decode_case(case, dev, kd, ops.Budget.ratio_budget(ratio, bos, 1), forced=forced,
                        check_dense=ratio == 0.125)
    n = case.n_chunks()
    for b in range(case.batch):
        K = min(int(n[b]), max(2 + bos, int(math.floor(int(n[b]) * ratio))))
        assert np.all(r["cnt"][b] == K)
        for h in range(case.num_kv_heads):
            s = r["sel"][b, h, :K]
            assert int(n[b]) - 1 in s and (not bos or 0 in s)


@pytest.mark.parametrize("which", ["1x32k-top256", "16x32k-top256", "64q-8kv-16x32k-ratio-1/8"])
def test_benchmark_decode_workloads_full_size(dev, which):
    """The benchmark's decode records at their own sizes and in the launch
    configuration it times (automatic splits; the fused call on its split
    grid): one sequence of 32,768 tokens with the 4096-token budget, the same
    layer over 16 sequences, and 64 q / 8 KV heads over 16 x 32,768 tokens at
    ratio 1/8 with bos + eos.  Full parity against the oracle: metadata,
    scores, selection (exact on the GPU's scores, band rule on the oracle's),
    attention; dense attention too at one sequence."""
    from block_sparse_attention_chunk_amd import ops
    if which == "1x32k-top256":
        case, kind, budget, forced = synth.replay_decode(seq_len=32768), ops.BSA_ENVELOPE, ops.Budget.topk(256), ()
    elif which == "16x32k-top256":
        case, kind, budget, forced = (synth.replay_decode(seq_len=32768, batch=16), ops.BSA_ENVELOPE,
                                      ops.Budget.topk(256), ())
    else:
        case, kind, budget, forced = (synth.batched_decode(cid=3, seq_lens=[32768] * 16), ops.BSA_CENTROID,
                                      ops.Budget.ratio_budget(0.125, 1, 1), ("bos", "eos"))
    r = run_decode_case(case, dev, kind, budget, forced=forced, check_dense=which == "1x32k-top256")
    assert np.all(r["cnt"] == budget.max_selected(2048))


@pytest.mark.parametrize("budget_kind", ["top-256", "ratio-1/16"])
def test_rows_longer_than_the_fused_selection(dev, budget_kind):
    """262,144 cached tokens (16,384 pages) at one sequence: the selection
    kernel takes rows of up to 16,384 candidates, and the fused entry point,
    whose own kernel selects at most 8,192, runs that selection kernel and
    then the split-grid attention -- bit-identical to the two calls.  Full
    parity against the oracle, dense attention included."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.replay_decode(cid=17, seq_len=262144)
    budget = ops.Budget.topk(256) if budget_kind == "top-256" else ops.Budget.ratio_budget(0.0625, 0, 1)
    forced = () if budget_kind == "top-256" else ("eos",)
    r = run_decode_case(case, dev, ops.BSA_ENVELOPE, budget, forced=forced, check_dense=budget_kind == "top-256")
    assert np.all(r["cnt"] == budget.max_selected(16384))


@pytest.mark.parametrize("dtype,D,hq", [("bf16", 128, 8), ("f32", 64, 8), ("bf16", 64, 32), ("f32", 128, 32)])
def test_balanced_schedule_edges(dev, dtype, D, hq):
    """The balanced schedule (automatic splits, 16 rows with room for 4096
    kept pages) on hand-made selections: one row keeping all 2048 pages of a 32K
    sequence (its positions fall into 128 workgroup shares, so its merge takes
    more than 64 partials), empty rows (0/0 = NaN, as in the oracle),
    single-page rows and partial last pages; query groups of 4 and 16 heads.
    Against the oracle; two calls give the same bits."""
    from block_sparse_attention_chunk_amd import ops
    case, sel, cnt = unequal_rows_case(21, synth.BF16 if dtype == "bf16" else synth.F32, D, 2101, hq)
    max_sel = sel.shape[2]
    log(f"case {case.name}: counts {cnt.tolist()}")
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    sel_t, cnt_t = ops.upload(sel, dev), ops.upload(cnt, dev)
    # the automatic call takes the balanced schedule: a workspace sized for the
    # split grid alone is refused
    g = hq // 2
    grid = ops.decode_num_splits(kv, hq, max_sel)
    small = torch.zeros((8 * hq * grid * (D + 2) * 4,), dtype=torch.uint8, device=dev)
    assert ops.decode_workspace_bytes(kv, hq, max_sel) == (16 + 256) * g * (D + 2) * 4 + 16 * (max_sel + 1) * 4
    assert (16 + 256) * g * (D + 2) * 4 > small.numel()
    with pytest.raises(RuntimeError, match="workspace"):
        ops.sparse_attn_decode(q, kv, sel_t, cnt_t, workspace=small)
    out1 = _np(ops.sparse_attn_decode(q, kv, sel_t, cnt_t))
    out2 = _np(ops.sparse_attn_decode(q, kv, sel_t, cnt_t))
    assert np.array_equal(out1, out2, equal_nan=True)
    ref = oracle.decode_attn(case.q, oracle_cache(case), sel, cnt)
    empty = np.repeat(cnt == 0, g, axis=1)                     # [B][H_q]
    assert np.all(np.isnan(out1[empty])) and np.all(np.isnan(ref[empty]))
    err = max_abs(out1[~empty], ref[~empty])
    log(f"  ok: attn err {err:.2e}")
    assert err <= ATTN_ABS[dtype]


def test_balanced_schedule_4096_rows(dev):
    """The balanced schedule at its row limit: 512 sequences x 8 KV heads =
    4096 rows (the counts' prefix is built in 16 rounds of 256 rows), lengths
    U[1, 256] tokens, random kept sets of 0-16 pages per row; against the
    oracle.  One row more and the call keeps the split grid."""
    from block_sparse_attention_chunk_amd import ops
    gen = np.random.default_rng(2301)
    B, H, D = 512, 8, 64
    lens = gen.integers(1, 257, size=B)
    case = synth.make_decode(23, batch=B, seq_lens=lens, num_q_heads=H, num_kv_heads=H, head_dim=D,
                             dtype=synth.BF16, name="balanced-4096-rows")
    max_sel = 16
    sel = np.full((B, H, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        pages = (int(lens[b]) + 15) // 16
        for h in range(H):
            c = int(gen.integers(0, pages + 1))
            cnt[b, h] = c
            sel[b, h, :c] = np.sort(gen.choice(pages, size=c, replace=False))
    kv, _ = gpu_kv(case, dev)
    assert ops.decode_workspace_bytes(kv, H, max_sel) == (4096 + 256) * 1 * (D + 2) * 4 + 4096 * (max_sel + 1) * 4
    out = _np(ops.sparse_attn_decode(ops.upload(case.q, dev), kv, ops.upload(sel, dev), ops.upload(cnt, dev)))
    ref = oracle.decode_attn(case.q, oracle_cache(case), sel, cnt)
    empty = cnt == 0
    assert np.all(np.isnan(out[empty])) and np.all(np.isnan(ref[empty]))
    err = max_abs(out[~empty], ref[~empty])
    log(f"  4096 rows: {int(empty.sum())} empty, attn err {err:.2e}")
    assert err <= ATTN_ABS["bf16"]


def test_partials_then_merge_matches_one_call(dev):
    """out == NULL leaves the split partials in the workspace; bsa_decode_merge
    on them gives the same bits as the single call (unfused and fused)."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.batched_decode(cid=15, batch=3, lo=1500, hi=4000)
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    meta = ops.build_chunk_meta(kv)
    sc = ops.score_chunks(q, kv, meta, ops.BSA_CENTROID)
    bud = ops.Budget.ratio_budget(0.25, 1, 1)
    sel, cnt = ops.select_topk(sc, kv, bud)
    B, Hq, D = case.batch, case.num_q_heads, case.head_dim
    for splits in (2, 5, 64):
        ws = torch.zeros((ops.decode_workspace_bytes(kv, Hq, int(sel.shape[2]), splits),), dtype=torch.uint8,
                         device=dev)
        full = ops.sparse_attn_decode(q, kv, sel, cnt, num_splits=splits)
        ops.sparse_attn_decode(q, kv, sel, cnt, num_splits=splits, out=ops.PARTIALS, workspace=ws)
        merged = ops.decode_merge(ws, B, Hq, D, splits)
        ws.zero_()
        ops.select_attn_decode(q, kv, sc, bud, num_splits=splits, out=ops.PARTIALS, workspace=ws)
        fmerged = ops.decode_merge(ws, B, Hq, D, splits)
        torch.cuda.synchronize()
        assert torch.equal(full, merged), splits
        assert torch.equal(full, fmerged), splits
    ref = oracle.decode_attn(case.q, oracle_cache(case), _np(sel), _np(cnt))
    assert max_abs(_np(full), ref) <= ATTN_ABS["bf16"]


def test_fused_token_budget_fixed_pages(dev):
    """Token budget over fixed pages (last page shorter) through the fused
    entry point: kept set equals the oracle's on the same scores."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(16, batch=3, seq_lens=[1000, 2049, 4100], num_q_heads=32, num_kv_heads=4,
                             head_dim=128, name="tokens-fixed")
    run_decode_case(case, dev, ops.BSA_ENVELOPE, ops.Budget.token_budget(1000), band_exact_count=False,
                    splits=(0, 3), check_dense=False)


@pytest.mark.parametrize("k", [64, 32])
def test_varchunk_centroid_topk(dev, k):
    """TSA chunking with centroid scoring and a chunk-count budget (top_k
    chunks per KV head, the tk64 / tk32 variants)."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.varchunk_decode()
    r = run_decode_case(case, dev, ops.BSA_CENTROID, ops.Budget.topk(k), check_dense=False, splits=(0, 5))
    assert np.all(r["cnt"] == k)


@pytest.mark.parametrize("seq_len,kind_budget", [(40000, "topk"), (120000, "ratio")])
def test_fused_long_rows(dev, seq_len, kind_budget):
    """Rows longer than 2048 pages: the fused kernel's wider per-thread
    candidate sets (one sequence, so the 8-wave selection) against the oracle
    and, bit for bit, against the two-call path."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(17, batch=1, seq_lens=[seq_len], num_q_heads=8, num_kv_heads=2, head_dim=128,
                             needles=12, name=f"long-{seq_len}")
    budget = ops.Budget.topk(300) if kind_budget == "topk" else ops.Budget.ratio_budget(1 / 16, 1, 1)
    forced = () if kind_budget == "topk" else ("bos", "eos")
    run_decode_case(case, dev, ops.BSA_ENVELOPE, budget, forced=forced, splits=(0, 7), check_dense=False)


@pytest.mark.parametrize("seq_len,kind_budget", [(40000, "topk"), (70000, "ratio")])
def test_fused_long_rows_large_grid(dev, seq_len, kind_budget):
    """Rows of 2,500 and 4,375 pages on a grid of more than one workgroup
    per compute unit (4 sequences x 4 KV heads x 17 splits): the fused
    kernel's 4-wave form with 16 and 32 candidates per thread, against the
    oracle and, bit for bit, against the two-call path."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(18, batch=4, seq_lens=[seq_len, seq_len - 999, seq_len // 2, seq_len - 16],
                             num_q_heads=8, num_kv_heads=4, head_dim=128, channel_scale=(0.5, 4.0),
                             name=f"long-grid-{seq_len}")
    budget = ops.Budget.topk(300) if kind_budget == "topk" else ops.Budget.ratio_budget(1 / 16, 1, 1)
    forced = () if kind_budget == "topk" else ("bos", "eos")
    run_decode_case(case, dev, ops.BSA_ENVELOPE, budget, forced=forced, splits=(17,), check_dense=False)


@pytest.mark.parametrize("fused", [False, True])
def test_empty_and_tiny_sequences(dev, fused):
    """Degenerate rows: a sequence with no cached token (no chunk to keep: the
    softmax over an empty set is 0/0, NaN, as in the oracle), a one-token
    sequence and budgets larger than a row (every chunk kept)."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(61, batch=4, seq_lens=[0, 100, 1, 37], num_q_heads=8, num_kv_heads=2, head_dim=128,
                             name="edge")
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    meta = ops.build_chunk_meta(kv)
    scores = ops.score_chunks(q, kv, meta, ops.BSA_ENVELOPE)
    budget = ops.Budget.topk(3)
    if fused:
        sel = torch.full((4, 2, 3), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((4, 2), -7, dtype=torch.int32, device=dev)
        out = ops.select_attn_decode(q, kv, scores, budget, num_splits=2, sel_idx=sel, sel_count=cnt)
    else:
        sel, cnt = ops.select_topk(scores, kv, budget)
        out = ops.sparse_attn_decode(q, kv, sel, cnt, num_splits=2)
    torch.cuda.synchronize()
    sc, sel, cnt, out = _np(scores), _np(sel), _np(cnt), _np(out)
    assert np.all(sc[0] == -np.inf)                              # no chunk in the empty row
    assert np.array_equal(cnt, [[0, 0], [3, 3], [1, 1], [3, 3]])
    assert np.all(sel[0] == -1) and np.all(sel[2, :, 1:] == -1)
    rsel, rcnt = oracle_select(sc.astype(np.float64), case, budget)
    assert np.array_equal(cnt, rcnt)
    oc = oracle_cache(case)
    ref = oracle.decode_attn(case.q, oc, sel, cnt)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(ref[0]))
    assert max_abs(out[1:], ref[1:]) <= ATTN_ABS[case.dtype]


def _clamp_case(case, sel, cnt, max_sel, rows):
    """Corrupt a valid selection the way a careless caller could, so that the
    clamped selection has no repeated page: rows = (full, no_first, no_last,
    negative) name the rows that get a count past max_sel (their list is full),
    a negative id (page 0 is not in their list), an id past the row (the last
    page is not in their list) and a negative count.  Returns the corrupted
    (sel, cnt) and the clamped equivalent the kernels must attend to."""
    n = case.n_chunks()
    bad_sel, bad_cnt = sel.copy(), cnt.copy()
    full, no_first, no_last, neg = rows
    gen = np.random.default_rng(len(sel.shape) + int(n.sum()))
    for b, h in (no_first, no_last):   # lists without the row's first and last page
        k = int(cnt[b, h])
        bad_sel[b, h, :k] = np.sort(gen.choice(np.arange(1, n[b] - 1), size=k, replace=False))
    sel = bad_sel.copy()
    if full is not None:
        b, h = full
        assert cnt[b, h] == max_sel
        bad_cnt[b, h] = max_sel + 9
    b, h = no_first
    assert cnt[b, h] >= 2 and 0 not in sel[b, h, :cnt[b, h]]
    bad_sel[b, h, 0] = -7
    b, h = no_last
    assert cnt[b, h] >= 2 and n[b] - 1 not in sel[b, h, :cnt[b, h]]
    bad_sel[b, h, cnt[b, h] - 1] = n[b] + 1000003
    b, h = neg
    bad_cnt[b, h] = -4
    want_cnt = np.clip(bad_cnt, 0, max_sel).astype(np.int32)
    want_sel = bad_sel.copy()
    for b in range(case.batch):
        for h in range(case.num_kv_heads):
            k = want_cnt[b, h]
            want_sel[b, h, :k] = np.clip(bad_sel[b, h, :k], 0, n[b] - 1)
    return bad_sel, bad_cnt, want_sel, want_cnt


@pytest.mark.parametrize("schedule", ["split-grid", "balanced", "segments", "per-token"])
def test_out_of_range_selection_is_clamped(dev, schedule):
    """Kept-page ids outside their row (negative, past the last page) and
    counts outside [0, max_sel] in a caller's selection are clamped into range
    by every decode schedule (the 16-token split grid, the balanced schedule,
    the 16-token-segment kernel for 32-token pages, the per-token kernel for
    8-token pages) rather than dereferenced: the output equals the oracle's on
    the clamped selection, and a row whose count clamps to 0 is empty (NaN)."""
    from block_sparse_attention_chunk_amd import ops
    if schedule == "balanced":
        case, sel, cnt = unequal_rows_case(23, synth.BF16, 128, 2102)
        max_sel, splits = sel.shape[2], 0
        rows = (None, (7, 1), (4, 1), (1, 0))
    else:
        page = {"split-grid": 16, "segments": 32, "per-token": 8}[schedule]
        case = synth.make_decode(70 + page, batch=2, seq_lens=[300, 1001], num_q_heads=8, num_kv_heads=2,
                                 head_dim=128, page_size=page, name=f"clamp-page{page}")
        n = case.n_chunks()
        max_sel = min(8, int(n.min()) - 1)
        gen = np.random.default_rng(page)
        sel = np.full((2, 2, max_sel), -1, np.int32)
        cnt = np.full((2, 2), max_sel, np.int32)
        for b in range(2):
            for h in range(2):
                pool = np.arange(1, n[b] - 1) if (b, h) != (0, 0) else np.arange(n[b])
                sel[b, h] = np.sort(gen.choice(pool, size=max_sel, replace=False))
        splits = 2
        rows = ((0, 0), (0, 1), (1, 0), (1, 1))
    log(f"clamped selection, schedule {schedule}")
    bad_sel, bad_cnt, want_sel, want_cnt = _clamp_case(case, sel, cnt, max_sel, rows)
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    out = _np(ops.sparse_attn_decode(q, kv, ops.upload(bad_sel, dev), ops.upload(bad_cnt, dev),
                                     num_splits=splits))
    torch.cuda.synchronize()
    ref = oracle.decode_attn(case.q, oracle_cache(case), want_sel, want_cnt)
    g = case.num_q_heads // case.num_kv_heads
    empty = np.repeat(want_cnt == 0, g, axis=1)
    assert np.all(np.isnan(out[empty])) and np.all(np.isnan(ref[empty]))
    err = max_abs(out[~empty], ref[~empty])
    assert err <= ATTN_ABS[case.dtype], err


def _random_config(i):
    """The i-th seeded configuration of the randomized sweep: shapes, dtype,
    page size, ragged lengths, scoring, budget and split count drawn
    together, so that combinations the fixed cases do not pair up are met."""
    r = np.random.default_rng(9000 + i)
    hkv = int(r.choice([1, 2, 3, 4]))
    g = int(r.choice([1, 2, 3, 4, 5, 7, 8, 11, 16]))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f32"]))
    page = int(r.choice([16, 16, 16, 32, 64]))
    batch = int(r.integers(1, 6))
    lens = [int(x) for x in r.integers(1, 6000, size=batch)]
    kind = str(r.choice(["envelope", "centroid"]))
    budget = str(r.choice(["topk", "ratio", "tokens"]))
    splits = int(r.choice([0, 0, 1, 2, 5, 13]))
    return dict(hkv=hkv, g=g, D=D, dtype=dtype, page=page, batch=batch, lens=lens, kind=kind, budget=budget,
                splits=splits)


@pytest.mark.parametrize("i", range(16))
def test_randomized_decode_configurations(dev, i):
    """Seeded random decode configurations, each through the full oracle
    comparison (metadata, scores, selection exact on the GPU's scores and by
    the band rule on the oracle's, attention, dense attention, the fused call
    bit for bit against the two calls on 16-token pages)."""
    from block_sparse_attention_chunk_amd import ops
    c = _random_config(i)
    log(f"random config {i}: {c}")
    case = synth.make_decode(9100 + i, batch=c["batch"], seq_lens=c["lens"], num_q_heads=c["hkv"] * c["g"],
                             num_kv_heads=c["hkv"], head_dim=c["D"], page_size=c["page"], dtype=c["dtype"],
                             channel_scale=(0.5, 4.0), name=f"random-{i}")
    n_max = int(max((L + c["page"] - 1) // c["page"] for L in c["lens"]))
    kd = ops.BSA_ENVELOPE if c["kind"] == "envelope" else ops.BSA_CENTROID
    forced = ()
    if c["budget"] == "topk":
        budget = ops.Budget.topk(max(1, n_max // 5))
    elif c["budget"] == "ratio":
        budget = ops.Budget.ratio_budget(0.25, 1, 1)
        forced = ("bos", "eos")
    else:
        budget = ops.Budget.token_budget(max(c["page"], n_max * c["page"] // 4))
    splits = (0, c["splits"]) if c["splits"] else (0,)
    run_decode_case(case, dev, kd, budget, forced=forced, splits=splits, band_exact_count=c["budget"] != "tokens")
