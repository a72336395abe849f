"""The C ABI's stream contract on the GPU: every call only enqueues on the
stream it is given (here torch's current stream), so the path runs on a side
stream and inside a captured HIP graph.

A graph of the decode step (scores, fused selection + attention, merge), one
of the balanced decode schedule and one of the router prefill (tile scores,
router, tile attention) are each replayed three times, with unrelated eager work on the same buffers and a
synchronisation between replays; every replay must give the eager result bit
for bit.  The library records no memset and allocates nothing, so a replay
redoes exactly the eager work.
"""
import numpy as np
import pytest

from block_sparse_attention_chunk_amd import synth
from parity_lib import gpu_kv, log, unequal_rows_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_chunk_amd import _abi
    _abi.lib()
    return torch.device("cuda:0")


def _decode_setup(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.replay_decode(cid=7, seq_len=6000)
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    meta = ops.build_chunk_meta(kv)
    budget = ops.Budget.topk(64)
    K = budget.max_selected(kv.max_pages)
    ws = torch.zeros((max(ops.decode_workspace_bytes(kv, case.num_q_heads, K), 16),), dtype=torch.uint8, device=dev)
    scores = torch.empty((1, case.num_kv_heads, kv.max_pages), dtype=torch.float32, device=dev)
    out = torch.empty((1, case.num_q_heads, case.head_dim), dtype=torch.float32, device=dev)

    def step():
        ops.score_chunks(q, kv, meta, ops.BSA_ENVELOPE, out=scores)
        ops.select_attn_decode(q, kv, scores, budget, out=out, workspace=ws)
    return step, out, scores


def test_decode_on_a_side_stream(dev):
    step, out, _ = _decode_setup(dev)
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)   # default priority
    with torch.cuda.stream(side):
        step()
    side.synchronize()
    assert torch.equal(out, ref)


def test_decode_graph_replays_match_eager(dev):
    step, out, scores = _decode_setup(dev)
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()                                  # warm-up on the capture stream
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        scores.fill_(0.0)                       # eager work on the graph's buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"decode graph replay {rep}")
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"


def test_balanced_decode_graph_replays_match_eager(dev):
    """The balanced decode schedule (16 rows of very unequal length,
    automatic splits) captured and replayed; between replays the workspace is
    cleared, so a replay must not depend on what an earlier call left there."""
    from block_sparse_attention_chunk_amd import ops
    case, sel, cnt = unequal_rows_case(22, synth.BF16, 128, 2201)
    kv, _ = gpu_kv(case, dev)
    q, sel_t, cnt_t = ops.upload(case.q, dev), ops.upload(sel, dev), ops.upload(cnt, dev)
    ws = torch.zeros((ops.decode_workspace_bytes(kv, 8, sel.shape[2]),), dtype=torch.uint8, device=dev)
    out = torch.empty((8, 8, 128), dtype=torch.float32, device=dev)

    def attend():
        ops.sparse_attn_decode(q, kv, sel_t, cnt_t, out=out, workspace=ws)

    attend()
    torch.cuda.synchronize()
    ref = out.cpu().numpy()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        attend()
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attend()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"balanced decode graph replay {rep}")
        assert np.array_equal(out.cpu().numpy(), ref, equal_nan=True), f"replay {rep} differs from the eager result"


def test_router_prefill_graph_replays_match_eager(dev):
    from block_sparse_attention_chunk_amd import ops
    pc = synth.router_prefill(cid=106, T=4096, k=8, groups=8, tied_groups=(1, 3, 5, 7))
    kv = ops.KVCache(ops.upload(pc.k, dev), ops.upload(pc.v, dev),
                     torch.tensor([pc.T], dtype=torch.int32, device=dev), pc.block, token_major=True)
    q = ops.upload(pc.q, dev)
    meta = ops.build_chunk_meta(kv)
    nt = (pc.T + pc.tile - 1) // pc.tile
    ts = torch.empty((nt, pc.num_kv_heads, kv.max_pages), dtype=torch.float32, device=dev)
    rws = torch.empty((max(ops.router_workspace_bytes(nt, pc.num_kv_heads, 8, 2), 16),), dtype=torch.uint8,
                      device=dev)
    pws = torch.empty((ops.tile_prefill_workspace_bytes(kv, pc.T),), dtype=torch.uint8, device=dev)
    out = torch.empty((pc.T, pc.num_q_heads, pc.head_dim), dtype=torch.float32, device=dev)
    held = {}

    def prefill():
        ops.score_chunks(q, kv, meta, ops.BSA_ENVELOPE, rows_per_query=pc.tile, causal=True, out=ts)
        held["r"] = ops.select_topk_router(ts, k=8, rho=2, workspace=rws)
        ops.sparse_attn_tile_prefill(q, kv, held["r"]["kv_idx"], out=out, workspace=pws)

    prefill()
    torch.cuda.synchronize()
    ref, ref_idx = out.clone(), held["r"]["kv_idx"].clone()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        prefill()
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prefill()
    torch.cuda.synchronize()
    cap_idx = held["r"]["kv_idx"]               # the graph's own output tensor
    for rep in range(3):
        out.fill_(float("nan"))
        ts.fill_(0.0)
        cap_idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"prefill graph replay {rep}")
        assert torch.equal(cap_idx, ref_idx), f"replay {rep}: router lists differ"
        assert torch.equal(out, ref), f"replay {rep}: tile attention differs from the eager result"
        assert np.isfinite(out.cpu().numpy()).all()
