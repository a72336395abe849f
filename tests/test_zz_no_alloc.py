"""The no-allocation fused decode entry point, bsa_select_attn_decode_static,
called through the C ABI: its output must equal bsa_select_attn_decode's
(same kernels, so bit for bit, which is within the 2e-3 max-abs attention
bound) on two calls in a row, the second on a smaller input, so stale
scratch contents from the first call cannot leak into the second."""
import ctypes

import numpy as np
import pytest

from block_sparse_attention_chunk_amd import synth
from parity_lib import ATTN_ABS, gpu_kv, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_chunk_amd import _abi
    _abi.lib()
    return torch.device("cuda:0")


def _static_call(q, kv, scores, budget, out):
    from block_sparse_attention_chunk_amd import _abi
    L = _abi.lib()
    rc = L.bsa_select_attn_decode_static(ctypes.c_void_p(q.data_ptr()), q.shape[1], ctypes.byref(kv.struct()),
                                         ctypes.c_void_p(scores.data_ptr()), ctypes.byref(budget.struct()),
                                         float(1.0 / np.sqrt(q.shape[2])), 0, ctypes.c_void_p(out.data_ptr()),
                                         None, None, 0,
                                         ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream))
    _abi.check(rc, "bsa_select_attn_decode_static")


def _run(case, dev, kind, budget):
    from block_sparse_attention_chunk_amd import ops
    kv, _ = gpu_kv(case, dev)
    q = ops.upload(case.q, dev)
    meta = ops.build_chunk_meta(kv)
    scores = ops.score_chunks(q, kv, meta, kind)
    K = budget.max_selected(kv.max_pages)
    need = ops.decode_workspace_bytes(kv, case.num_q_heads, K)
    assert 0 < need <= 16 << 20
    ref = ops.select_attn_decode(q, kv, scores, budget)
    out = torch.full_like(ref, float("nan"))
    _static_call(q, kv, scores, budget, out)
    torch.cuda.synchronize()
    err = float((out - ref).abs().max())
    assert err <= ATTN_ABS[case.dtype], err
    assert torch.equal(out, ref), "static-scratch output differs from the workspace call"
    return need


def test_static_scratch_two_calls_second_smaller(dev):
    from block_sparse_attention_chunk_amd import ops
    # 1: the ragged 16-sequence batch at ratio 1/2 (selection kernel + the
    # balanced attention, ~2 MB of scratch)
    big = synth.batched_decode()
    log("static scratch, call 1: 16 x U[8K, 32K] tokens, 64 q / 8 KV heads, ratio 1/2")
    n1 = _run(big, dev, ops.BSA_CENTROID, ops.Budget.ratio_budget(0.5, 1, 1))
    # 2: one 6,000-token replay-shaped sequence, top-64 pages (the fused
    # kernel with split partials, a smaller part of the scratch)
    small = synth.replay_decode(cid=7, seq_len=6000)
    log("static scratch, call 2: 1 x 6000 tokens, 32 q / 4 KV heads, top-64")
    n2 = _run(small, dev, ops.BSA_ENVELOPE, ops.Budget.topk(64))
    assert n2 < n1
    log(f"  ok: scratch bytes {n1} then {n2}")
