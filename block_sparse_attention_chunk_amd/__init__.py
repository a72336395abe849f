"""Query-aware block-sparse attention over a chunked, paged GQA KV cache for
AMD Instinct MI355X (gfx950): the C-ABI library libbsa.so (hand-written HIP)
and its Python binding.

    from block_sparse_attention_chunk_amd import ops
    meta = ops.build_chunk_meta(kv)
    scores = ops.score_chunks(q, kv, meta, ops.BSA_ENVELOPE)
    sel_idx, sel_count = ops.select_topk(scores, kv, ops.Budget.topk(256))
    out = ops.sparse_attn_decode(q, kv, sel_idx, sel_count)
"""
