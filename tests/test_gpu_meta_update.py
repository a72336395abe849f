"""Incremental chunk metadata (bsa_update_chunk_meta) against a full rebuild
(bsa_build_chunk_meta, itself oracle-checked in the decode parity tests):
after appending tokens -- one at a time, or several at once -- every chunk's
kmin / kmax / centroid must be bit-identical to a rebuild at the new length.
Fixed 16-token pages with a shuffled block table, and variable chunks whose
last chunk grows."""
import numpy as np
import pytest

from block_sparse_attention_chunk_amd import synth
from parity_lib import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_chunk_amd import _abi
    _abi.lib()
    return torch.device("cuda:0")


def _kv(ops, case, dev, lens):
    return ops.KVCache(ops.upload(case.k, dev), ops.upload(case.v, dev), torch.tensor(lens, dtype=torch.int32,
                       device=dev), case.page_size, ops.upload(case.block_table, dev))


def _same(a, b, n):
    for x, y in ((a.kmin, b.kmin), (a.kmax, b.kmax), (a.centroid, b.centroid)):
        for bi, nb in enumerate(n):
            assert torch.equal(x[bi, :, :nb], y[bi, :, :nb])


def test_append_one_token_at_a_time(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(50, batch=3, seq_lens=[100, 513, 1040], num_q_heads=8, num_kv_heads=2, head_dim=128,
                             name="append")
    L = np.array(case.seq_lens)
    L0 = L - np.array([20, 37, 5])
    log("append one token at a time")
    kv0 = _kv(ops, case, dev, L0)
    meta = ops.build_chunk_meta(kv0)
    cur = L0.copy()
    while (cur < L).any():
        cur = np.minimum(cur + 1, L)
        ops.update_chunk_meta(_kv(ops, case, dev, cur), meta)      # last chunk only
    ref = ops.build_chunk_meta(_kv(ops, case, dev, L))
    torch.cuda.synchronize()
    _same(meta, ref, (L + 15) // 16)


@pytest.mark.parametrize("dtype_f32", [False, True])
def test_append_many_tokens(dev, dtype_f32):
    from block_sparse_attention_chunk_amd import ops
    case = synth.make_decode(51, batch=4, seq_lens=[64, 700, 1999, 3000], num_q_heads=4, num_kv_heads=2,
                             head_dim=64, dtype="f32" if dtype_f32 else "bf16", name="append-many")
    L = np.array(case.seq_lens)
    L0 = np.array([0, 650, 1900, 3000])          # empty start, several pages, no change
    log(f"append many tokens (f32={dtype_f32})")
    meta = ops.build_chunk_meta(_kv(ops, case, dev, np.maximum(L0, 1)))
    kv = _kv(ops, case, dev, L)
    a = int((L - L0).max())
    ops.update_chunk_meta(kv, meta, from_len=torch.tensor(L0, dtype=torch.int32, device=dev),
                          max_touched=(a + 15) // 16 + 1)
    ref = ops.build_chunk_meta(kv)
    torch.cuda.synchronize()
    _same(meta, ref, (L + 15) // 16)


def test_variable_chunks_last_chunk_grows(dev):
    from block_sparse_attention_chunk_amd import ops
    case = synth.varchunk_decode(cid=2, seq_len=4000)
    starts = case.chunk_starts.copy()
    n = int(case.num_chunks[0])
    L = int(case.seq_lens[0])
    last_start = int(starts[0, n - 1])
    L0 = last_start + 1                      # the last chunk had one token
    log("variable chunks: last chunk grows")
    st0 = starts.copy()
    st0[0, n] = L0
    kv0 = _kv(ops, case, dev, [L0])
    ch0 = ops.Chunks(ops.upload(st0, dev), ops.upload(case.num_chunks, dev))
    meta = ops.build_chunk_meta(kv0, ch0)
    kv = _kv(ops, case, dev, [L])
    ch = ops.Chunks(ops.upload(starts, dev), ops.upload(case.num_chunks, dev))
    ops.update_chunk_meta(kv, meta, chunks=ch, from_len=torch.tensor([L0], dtype=torch.int32, device=dev),
                          max_touched=1)
    ref = ops.build_chunk_meta(kv, ch)
    torch.cuda.synchronize()
    _same(meta, ref, [n])
