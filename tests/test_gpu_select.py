"""GPU selection on hand-made score rows full of ties, against the oracle's
selection on the same fp32 scores: the kept sets must be identical (the
selection is an exact function of its scores).  Rows of 300, 2048 and 5000
chunks exercise both workgroup sizes; every budget mode; rows of equal
scores; token weights from fixed pages with a short last page.  The fused
selection + decode entry point must keep the same lists."""
import numpy as np
import pytest

import oracle
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


def _case(seed, n_max, B=6, H=3):
    rng = np.random.default_rng(seed)
    n = rng.integers(max(1, n_max // 3), n_max + 1, B)
    n[0] = n_max
    lens = n * 16 - rng.integers(0, 16, B)
    sc = np.full((B, H, n_max), -np.inf, np.float32)
    for b in range(B):
        for h in range(H):
            if (b + h) % 5 == 0:
                sc[b, h, :n[b]] = 2.5                                # one big tie
            elif (b + h) % 2:
                sc[b, h, :n[b]] = rng.integers(-3, 4, n[b])          # few distinct values
            else:
                sc[b, h, :n[b]] = rng.normal(size=n[b]).astype(np.float32)
    return n, lens.astype(np.int32), sc


def _chunk_len(n, lens, n_max):
    cl = np.zeros((len(n), n_max), np.int32)
    for b in range(len(n)):
        cl[b, :n[b]] = 16
        cl[b, n[b] - 1] = lens[b] - 16 * (n[b] - 1)
    return cl


@pytest.mark.parametrize("n_max", [300, 2048, 5000, 12000])
@pytest.mark.parametrize("mode", ["topk", "tokens", "ratio_bos_eos", "ratio_eos"])
def test_selection_with_ties_is_exact(dev, n_max, mode):
    from block_sparse_attention_chunk_amd import ops
    n, lens, sc = _case(100 + n_max, n_max)
    B, H = sc.shape[:2]
    log(f"ties n_max={n_max} mode={mode}")
    dummy = torch.zeros((1, H, 16, 64), dtype=torch.bfloat16, device=dev)
    kv = ops.KVCache(dummy, dummy, torch.tensor(lens, device=dev), 16,
                     torch.zeros((B, n_max), dtype=torch.int32, device=dev))
    if mode == "topk":
        bud = ops.Budget.topk(max(1, n_max // 7))
        ref = oracle.select(sc.astype(np.float64), n, oracle.TOPK, top_k=bud.top_k, max_sel=n_max)
    elif mode == "tokens":
        bud = ops.Budget.token_budget(n_max * 3 + 5)
        ref = oracle.select(sc.astype(np.float64), n, oracle.TOKENS, tokens=bud.tokens,
                            chunk_len=_chunk_len(n, lens, n_max), max_sel=n_max)
    else:
        bos = 1 if mode == "ratio_bos_eos" else 0
        bud = ops.Budget.ratio_budget(0.125, bos, 1)
        ref = oracle.select(sc.astype(np.float64), n, oracle.RATIO, ratio=0.125, bos=bos, eos=1,
                            max_sel=n_max)
    scores = torch.tensor(sc, device=dev)
    sel, cnt = ops.select_topk(scores, kv, bud)
    # the fused selection + attention writes the same kept list: a small grid
    # (8 waves share the selection) and a large one (4 waves)
    q = torch.zeros((B, H, 64), dtype=torch.bfloat16, device=dev)
    fused = []
    for splits in (0, 64):
        fsel, fcnt = torch.full_like(sel, -7), torch.full_like(cnt, -7)
        ops.select_attn_decode(q, kv, scores, bud, num_splits=splits, sel_idx=fsel, sel_count=fcnt)
        fused.append((splits, fsel, fcnt))
    torch.cuda.synchronize()
    for splits, fsel, fcnt in fused:
        assert torch.equal(fsel, sel) and torch.equal(fcnt, cnt), f"fused selection differs (splits={splits})"
    sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    rsel, rcnt = ref
    assert np.array_equal(cnt, rcnt)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(sel[b, h, :cnt[b, h]], rsel[b, h, :rcnt[b, h]]), (b, h)
            assert np.all(sel[b, h, cnt[b, h]:] == -1)
