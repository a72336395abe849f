"""bsa_decode_step: the whole decode step in one call (scoring, then the
fused selection + attention and the split merge).  Its output, scores and
kept lists must be bit-identical to bsa_score_chunks + bsa_select_attn_decode
at the same split count, and the output must match the oracle's attention on
the kept lists.  Also: a workspace full of garbage (it needs no initial
contents), split counts from 2 to 64, a batch on the balanced schedule, and
HIP graph replays with eager work between them."""
import numpy as np
import pytest

import oracle
from block_sparse_attention_chunk_amd import synth
from parity_lib import ATTN_ABS, gpu_kv, log, max_abs, oracle_cache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_chunk_amd import _abi
    _abi.lib()
    return torch.device("cuda:0")


def _step_vs_two_calls(case, dev, kind, budget, splits=0, garbage=False, check_oracle=True):
    from block_sparse_attention_chunk_amd import ops
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    which = ops.BSA_META_ENVELOPE if kind == ops.BSA_ENVELOPE else ops.BSA_META_CENTROID
    meta = ops.build_chunk_meta(kv, which=which)
    K = budget.max_selected(kv.max_pages)
    B, H = case.batch, case.num_kv_heads
    need = ops.decode_step_workspace_bytes(kv, case.num_q_heads, budget, splits)
    ws = torch.full((need,), 0xFF if garbage else 0, dtype=torch.uint8, device=dev)
    sc = torch.full((B, H, kv.max_pages), 7.0, dtype=torch.float32, device=dev)
    sel = torch.full((B, H, K), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, H), -7, dtype=torch.int32, device=dev)
    out = ops.decode_step(q, kv, meta, kind, budget, num_splits=splits, scores=sc, workspace=ws, sel_idx=sel,
                          sel_count=cnt)
    # the two-call path at the same split count
    ref_sc = ops.score_chunks(q, kv, meta, kind)
    rsel = torch.full_like(sel, -7)
    rcnt = torch.full_like(cnt, -7)
    ref = ops.select_attn_decode(q, kv, ref_sc, budget, num_splits=splits, sel_idx=rsel, sel_count=rcnt)
    torch.cuda.synchronize()
    assert torch.equal(sc, ref_sc), "scores differ from bsa_score_chunks"
    assert torch.equal(sel, rsel) and torch.equal(cnt, rcnt), "kept lists differ from bsa_select_attn_decode"
    assert torch.equal(out, ref), "output not bit-identical to the two-call path"
    if check_oracle:
        o = oracle.decode_attn(case.q, oracle_cache(case), sel.cpu().numpy(), cnt.cpu().numpy())
        err = max_abs(out.cpu().numpy(), o)
        assert err <= ATTN_ABS[case.dtype], err
    return out


@pytest.mark.parametrize("which", ["tiny-f32", "replay-6000-top64", "replay-32k-top256", "batched-4x", "replay-256k-top256"])
def test_decode_step_matches_two_calls_and_oracle(dev, which):
    from block_sparse_attention_chunk_amd import ops
    if which == "tiny-f32":
        case, kind, budget = synth.tiny_decode(), ops.BSA_ENVELOPE, ops.Budget.topk(8)
    elif which == "replay-6000-top64":
        case, kind, budget = synth.replay_decode(cid=7, seq_len=6000), ops.BSA_CENTROID, ops.Budget.topk(64)
    elif which == "replay-32k-top256":
        case, kind, budget = synth.replay_decode(seq_len=32768), ops.BSA_ENVELOPE, ops.Budget.topk(256)
    elif which == "replay-256k-top256":     # rows longer than the fused kernel selects: two passes
        case, kind, budget = synth.replay_decode(cid=18, seq_len=262144), ops.BSA_CENTROID, ops.Budget.topk(256)
    else:
        case = synth.batched_decode(cid=15, batch=4, lo=3000, hi=9000)
        kind, budget = ops.BSA_ENVELOPE, ops.Budget.ratio_budget(0.125, 0, 1)
    log(f"decode step {which}")
    _step_vs_two_calls(case, dev, kind, budget)


@pytest.mark.parametrize("splits", [2, 7, 64])
def test_decode_step_split_counts_and_garbage_workspace(dev, splits):
    from block_sparse_attention_chunk_amd import ops
    case = synth.replay_decode(cid=8, seq_len=9000)
    log(f"decode step, {splits} splits, workspace filled with 0xff")
    _step_vs_two_calls(case, dev, ops.BSA_ENVELOPE, ops.Budget.topk(200), splits=splits, garbage=True)


def test_decode_step_balanced_batch(dev):
    """16 x U[8K, 32K] tokens, 64 q / 8 KV heads, ratio 1/2: the scoring, the
    selection kernel and the balanced attention (no in-launch merge)."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.batched_decode()
    log("decode step on the balanced schedule")
    _step_vs_two_calls(case, dev, ops.BSA_CENTROID, ops.Budget.ratio_budget(0.5, 1, 1), check_oracle=False)


def test_decode_step_graph_replays(dev):
    """A captured decode step replayed three times, with eager steps between
    the replays, gives the eager output each time."""
    from block_sparse_attention_chunk_amd import ops
    case = synth.replay_decode(cid=9, seq_len=12000)
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    meta = ops.build_chunk_meta(kv, which=ops.BSA_META_ENVELOPE)
    budget = ops.Budget.topk(128)
    ws = torch.empty((ops.decode_step_workspace_bytes(kv, case.num_q_heads, budget),), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((1, case.num_q_heads, case.head_dim), dtype=torch.float32, device=dev)
    eager = ops.decode_step(q, kv, meta, ops.BSA_ENVELOPE, budget, workspace=ws).clone()
    torch.cuda.synchronize()
    ops.decode_step(q, kv, meta, ops.BSA_ENVELOPE, budget, out=out, workspace=ws)   # loads the code objects
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.decode_step(q, kv, meta, ops.BSA_ENVELOPE, budget, out=out, workspace=ws)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager step"
        again = ops.decode_step(q, kv, meta, ops.BSA_ENVELOPE, budget, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)
