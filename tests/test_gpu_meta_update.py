"""Incremental chunk metadata (bsa_update_chunk_meta): after appending
tokens -- one at a time, or several at once -- every chunk's kmin / kmax /
centroid must be bit-identical to a full rebuild at the new length
(bsa_build_chunk_meta) and must match the oracle's metadata at the new length
directly (kmin / kmax bit-exact, centroid within the float32 summation
bound).  Fixed 16-token pages with a shuffled block table, and variable
chunks whose last chunk grows."""
import numpy as np
import pytest

import oracle
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


def _vs_oracle(meta, case, lens, starts=None, num=None):
    """The updated metadata against the oracle's metadata of the grown cache."""
    oc = oracle.PagedCache(case.k, case.v, case.block_table, lens, case.page_size, case.num_kv_heads, case.head_dim)
    omin, omax, ocen = oracle.chunk_meta(oc, starts, num)
    kmin, kmax = oracle.to_f64(_host(meta.kmin)), oracle.to_f64(_host(meta.kmax))
    cen = meta.centroid.cpu().numpy()
    kabs = float(np.nanmax(np.abs(oracle.to_f64(case.k))))
    longest = case.page_size if starts is None else int(np.max(np.diff(starts, axis=1)))
    tol = (longest + 1) * 2.0 ** -24 * kabs
    n = (np.asarray(lens) + case.page_size - 1) // case.page_size if starts is None else np.asarray(num)
    for b, nb in enumerate(n):
        nb = int(nb)
        assert np.array_equal(kmin[b, :, :nb], omin[b, :, :nb]), f"kmin of sequence {b} differs from the oracle"
        assert np.array_equal(kmax[b, :, :nb], omax[b, :, :nb]), f"kmax of sequence {b} differs from the oracle"
        assert np.max(np.abs(cen[b, :, :nb] - ocen[b, :, :nb])) <= tol, f"centroid of sequence {b}"


def _host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


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
    _vs_oracle(meta, case, L)


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
    _vs_oracle(meta, case, L)


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
    _vs_oracle(meta, case, [L], starts, case.num_chunks)


def _random_update_config(i):
    """The i-th seeded incremental-update case: chunking (fixed pages of 16,
    32 or 64 tokens, or variable chunks of 4-60 tokens), batch, heads, head
    dim, dtype, new lengths and the tokens appended per sequence."""
    r = np.random.default_rng(8000 + i)
    batch = int(r.integers(1, 5))
    L = r.integers(1, 3000, size=batch)
    a = np.minimum(r.integers(0, 300, size=batch), L - 1)      # at least one token was there before
    return dict(batch=batch, hkv=int(r.choice([1, 2, 4])), d=int(r.choice([64, 128])),
                f32=bool(r.integers(0, 2)), page=int(r.choice([16, 32, 64])), variable=bool(i % 2),
                L=L.astype(np.int32), L0=(L - a).astype(np.int32))


@pytest.mark.parametrize("i", range(8))
def test_randomized_updates(dev, i):
    """Seeded appends of 0-299 tokens per sequence: the chunks an update
    recomputes match a full rebuild bit for bit and the oracle's metadata of
    the grown cache (kmin / kmax bit-exact, centroid within the fp32 bound)."""
    from block_sparse_attention_chunk_amd import ops
    c = _random_update_config(i)
    B, L, L0 = c["batch"], c["L"], c["L0"]
    page = 16 if c["variable"] else c["page"]
    log(f"random update {i}: {c}")
    case = synth.make_decode(8100 + i, batch=B, seq_lens=L, num_q_heads=c["hkv"], num_kv_heads=c["hkv"],
                             head_dim=c["d"], page_size=page, dtype="f32" if c["f32"] else "bf16",
                             name=f"update-{i}")
    from_len = torch.tensor(L0, dtype=torch.int32, device=dev)
    if not c["variable"]:
        meta = ops.build_chunk_meta(_kv(ops, case, dev, L0))
        touched = int(np.max((L - L0 + page - 1) // page + 1))
        kv = _kv(ops, case, dev, L)
        ops.update_chunk_meta(kv, meta, from_len=from_len, max_touched=min(touched, kv.max_pages))
        ref = ops.build_chunk_meta(kv)
        torch.cuda.synchronize()
        _same(meta, ref, (L + page - 1) // page)
        _vs_oracle(meta, case, L)
        return
    # variable chunks: the grown layout, and the old one (its chunks that start
    # before the old length, the last one cut there)
    r = np.random.default_rng(8500 + i)
    new, old = [], []
    for b in range(B):
        s = [0]
        while s[-1] < L[b]:
            s.append(min(int(L[b]), s[-1] + int(r.integers(4, 61))))
        s = np.asarray(s, np.int32)
        n0 = int(np.searchsorted(s, L0[b], side="left"))        # chunks starting before L0
        o = np.concatenate([s[:n0], [L0[b]]]).astype(np.int32)
        new.append(s)
        old.append(o)
    synth.with_chunks(case, new)
    starts, num = case.chunk_starts, case.num_chunks
    mc = starts.shape[1] - 1
    st0 = np.zeros_like(starts)
    num0 = np.array([len(o) - 1 for o in old], np.int32)
    for b, o in enumerate(old):
        st0[b, :len(o)] = o
        st0[b, len(o):] = o[-1]
    touched = int(max(len(new[b]) - 1 - (len(old[b]) - 2) for b in range(B)))
    meta = ops.build_chunk_meta(_kv(ops, case, dev, L0), ops.Chunks(ops.upload(st0, dev), ops.upload(num0, dev)))
    kv = _kv(ops, case, dev, L)
    ch = ops.Chunks(ops.upload(starts, dev), ops.upload(num, dev))
    ops.update_chunk_meta(kv, meta, chunks=ch, from_len=from_len, max_touched=min(touched, mc))
    ref = ops.build_chunk_meta(kv, ch)
    torch.cuda.synchronize()
    _same(meta, ref, num)
    _vs_oracle(meta, case, L, starts, num)
