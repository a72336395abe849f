"""The C-ABI library on the CPU: it loads, exports every entry point that
include/bsa.h declares, and rejects invalid arguments on the host before any
HIP call (so no GPU is needed)."""
import ctypes
import math
import os
import re

import pytest

from block_sparse_attention_chunk_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 16-byte-aligned non-NULL address; never dereferenced by host validation


def _declared():
    src = open(os.path.join(ROOT, "include", "bsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_abi.SIGNATURES)


def test_status_strings():
    L = _abi.lib()
    for code, name in [(0, "BSA_OK"), (-1, "BSA_ERR_INVALID_ARG"), (-2, "BSA_ERR_UNSUPPORTED"),
                       (-3, "BSA_ERR_WORKSPACE"), (-4, "BSA_ERR_LAUNCH")]:
        assert L.bsa_status_string(code).decode() == name


def _kv(**over):
    d = dict(k=FAKE, v=FAKE, stride_page=2 * 16 * 128, stride_head=16 * 128, stride_token=128, block_table=FAKE,
             seq_lens=FAKE, batch=1, num_kv_heads=2, head_dim=128, page_size=16, max_pages=64, dtype=_abi.BSA_BF16)
    d.update(over)
    return _abi.bsa_kv(**d)


def _decode(kv, hq=8, sel=True, scale=0.088, splits=1, ws=None, ws_bytes=0, max_sel=8, count=True):
    L = _abi.lib()
    return L.bsa_sparse_attn_decode(FAKE, hq, ctypes.byref(kv), None, FAKE if sel else None,
                                    FAKE if count else None, max_sel, scale, splits, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("over,code,msg", [
    (dict(k=None), _abi.BSA_ERR_INVALID_ARG, "kv->k"),
    (dict(v=None), _abi.BSA_ERR_INVALID_ARG, "kv->v"),
    (dict(seq_lens=None), _abi.BSA_ERR_INVALID_ARG, "seq_lens"),
    (dict(head_dim=96), _abi.BSA_ERR_UNSUPPORTED, "head_dim"),
    (dict(page_size=24), _abi.BSA_ERR_UNSUPPORTED, "page_size"),
    (dict(page_size=512), _abi.BSA_ERR_UNSUPPORTED, "page_size"),
    (dict(dtype=7), _abi.BSA_ERR_UNSUPPORTED, "dtype"),
    (dict(k=FAKE + 2), _abi.BSA_ERR_INVALID_ARG, "aligned"),
    (dict(stride_token=100), _abi.BSA_ERR_INVALID_ARG, "strides"),
    (dict(batch=0), _abi.BSA_ERR_INVALID_ARG, "batch"),
])
def test_decode_rejects_bad_cache(over, code, msg):
    L = _abi.lib()
    assert _decode(_kv(**over)) == code
    assert msg in L.bsa_last_error().decode()


def test_decode_argument_checks():
    L = _abi.lib()
    assert _decode(_kv(), hq=7) == _abi.BSA_ERR_INVALID_ARG           # 7 % 2 != 0
    assert _decode(_kv(), hq=34) == _abi.BSA_ERR_UNSUPPORTED          # group 17 > 16
    assert _decode(_kv(), scale=0.0) == _abi.BSA_ERR_INVALID_ARG
    assert _decode(_kv(), scale=math.inf) == _abi.BSA_ERR_INVALID_ARG
    assert _decode(_kv(), count=False) == _abi.BSA_ERR_INVALID_ARG
    assert _decode(_kv(), splits=-1) == _abi.BSA_ERR_INVALID_ARG
    # 4 splits need a workspace of B*H_q*splits*(D+2)*4 bytes
    need = L.bsa_decode_workspace_bytes(ctypes.byref(_kv()), 8, 8, 4)
    assert need == 1 * 8 * 4 * 130 * 4
    assert _decode(_kv(), splits=4) == _abi.BSA_ERR_WORKSPACE
    assert _decode(_kv(), splits=4, ws=FAKE, ws_bytes=need - 1) == _abi.BSA_ERR_WORKSPACE
    assert "workspace" in L.bsa_last_error().decode()


def test_decode_split_resolution():
    L = _abi.lib()
    kv = _kv(batch=16, num_kv_heads=8)
    assert L.bsa_decode_num_splits(ctypes.byref(kv), 64, 256, 0) == 2        # ~256 workgroups
    assert L.bsa_decode_num_splits(ctypes.byref(kv), 64, 256, 5) == 5        # explicit
    kv16 = _kv(batch=16, num_kv_heads=4)
    assert L.bsa_decode_num_splits(ctypes.byref(kv16), 32, 256, 0) == 4
    kv1 = _kv(batch=1, num_kv_heads=4)
    assert L.bsa_decode_num_splits(ctypes.byref(kv1), 32, 256, 0) == 32      # capped at ~8 items per workgroup
    assert L.bsa_decode_num_splits(ctypes.byref(kv1), 32, 1844, 0) == 64      # the cap of 64 splits
    kv_many = _kv(batch=64, num_kv_heads=8)
    assert L.bsa_decode_num_splits(ctypes.byref(kv_many), 64, 256, 0) == 1   # enough rows: one split, no merge
    assert L.bsa_decode_num_splits(ctypes.byref(kv1), 32, 3, 0) == 1
    assert L.bsa_decode_workspace_bytes(ctypes.byref(kv1), 32, 3, 0) == 0


def test_balanced_schedule_workspace():
    """Automatic splits on batches of 16-token pages with enough work take the
    balanced schedule: 256 workgroup shares, one partial per (row, share) met,
    (rows + 256) x group entries of (D + 2) floats."""
    L = _abi.lib()
    kv = _kv(batch=16, num_kv_heads=8, max_pages=2048)
    split_bytes = 16 * 64 * 2 * 130 * 4                       # 2 automatic splits
    bal_bytes = (128 + 256) * 8 * 130 * 4
    lists = 128 * (946 + 1) * 4                               # kept lists of the fused entry point
    assert L.bsa_decode_workspace_bytes(ctypes.byref(kv), 64, 946, 0) == max(split_bytes, bal_bytes + lists)
    assert L.bsa_decode_workspace_bytes(ctypes.byref(kv), 64, 946, 2) == split_bytes   # explicit: split grid
    # 128 rows x 383 items < 192 x 256: the split grid only
    assert L.bsa_decode_workspace_bytes(ctypes.byref(kv), 64, 383, 0) == split_bytes
    assert L.bsa_decode_workspace_bytes(ctypes.byref(kv), 64, 384, 0) == max(split_bytes, bal_bytes + 128 * 385 * 4)
    # fewer than 16 rows: the split grid only
    kv8 = _kv(batch=4, num_kv_heads=2, max_pages=4096)
    s8 = L.bsa_decode_num_splits(ctypes.byref(kv8), 8, 4096, 0)
    assert L.bsa_decode_workspace_bytes(ctypes.byref(kv8), 8, 4096, 0) == 4 * 8 * s8 * 130 * 4
    # other page sizes keep the split grid
    kvp = _kv(batch=16, num_kv_heads=8, max_pages=2048, page_size=32, stride_page=2 * 32 * 128,
              stride_head=32 * 128)
    assert L.bsa_decode_workspace_bytes(ctypes.byref(kvp), 64, 946, 0) == split_bytes
    # the row limits: 16 to 4096 rows (batch x H_kv)
    def ws(batch, hkv, hq, items):
        return L.bsa_decode_workspace_bytes(ctypes.byref(_kv(batch=batch, num_kv_heads=hkv, max_pages=8192)), hq,
                                            items, 0)

    def grid_bytes(batch, hkv, hq, items):
        k = _kv(batch=batch, num_kv_heads=hkv, max_pages=8192)
        s = L.bsa_decode_num_splits(ctypes.byref(k), hq, items, 0)
        return 0 if s <= 1 else batch * hq * s * 130 * 4

    for batch, hkv, on in ((15, 1, False), (16, 1, True), (512, 8, True), (4097, 1, False)):
        items = 8192 if batch * hkv < 64 else 64
        bal = ((batch * hkv + 256) * 1 * 130 * 4 + 15) // 16 * 16 + batch * hkv * (items + 1) * 4
        want = max(grid_bytes(batch, hkv, hkv, items), bal) if on else grid_bytes(batch, hkv, hkv, items)
        assert ws(batch, hkv, hkv, items) == want, (batch, hkv)
    # the balanced call checks its own workspace size
    assert _decode(kv, hq=64, splits=0, max_sel=946, ws=FAKE, ws_bytes=bal_bytes - 1) == _abi.BSA_ERR_WORKSPACE
    assert "%d bytes" % bal_bytes in L.bsa_last_error().decode()
    # a chunk struct without chunk_starts means fixed pages: the same schedule
    empty = _abi.bsa_chunks(None, None, 0)
    rc = L.bsa_sparse_attn_decode(FAKE, 64, ctypes.byref(kv), ctypes.byref(empty), FAKE, FAKE, 946, 0.088, 0, FAKE,
                                  FAKE, bal_bytes - 1, None)
    assert rc == _abi.BSA_ERR_WORKSPACE
    assert "%d bytes" % bal_bytes in L.bsa_last_error().decode()


def _select(kv, budget, max_sel, chunks=None):
    L = _abi.lib()
    return L.bsa_select_topk(FAKE, ctypes.byref(kv), chunks, ctypes.byref(budget), FAKE, FAKE, max_sel, None)


def _golden(name):
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c.strip() for c in line.split(";")])
    return rows


def test_select_max_count_matches_the_ratio_budget_table():
    """bsa_select_max_count against the worked ratio-budget values
    (tests/golden/ratio_budget.txt), plus the top-k and token rules."""
    L = _abi.lib()
    B = _abi.bsa_budget
    rows = _golden("ratio_budget.txt")
    assert len(rows) >= 10
    for n, ratio, bos, eos, want in rows:
        b = B(_abi.BSA_BUDGET_RATIO, 0, 0, int(bos), int(eos), float(ratio))
        assert L.bsa_select_max_count(ctypes.byref(b), int(n)) == int(want), (n, ratio, bos, eos)
    assert L.bsa_select_max_count(ctypes.byref(B(_abi.BSA_BUDGET_TOPK, 256, 0, 0, 0, 0.0)), 1844) == 256
    assert L.bsa_select_max_count(ctypes.byref(B(_abi.BSA_BUDGET_TOPK, 256, 0, 0, 0, 0.0)), 100) == 100
    assert L.bsa_select_max_count(ctypes.byref(B(_abi.BSA_BUDGET_TOKENS, 0, 4096, 0, 0, 0.0)), 221) == 221
    assert L.bsa_select_max_count(ctypes.byref(B(_abi.BSA_BUDGET_TOKENS, 0, 40, 0, 0, 0.0)), 221) == 40
    # invalid budgets and sizes give error codes with a message
    for bad, n in [(B(_abi.BSA_BUDGET_TOPK, 0, 0, 0, 0, 0.0), 10), (B(_abi.BSA_BUDGET_RATIO, 0, 0, 0, 1, 0.0), 10),
                   (B(_abi.BSA_BUDGET_RATIO, 0, 0, 2, 1, 0.5), 10), (B(9, 1, 0, 0, 0, 0.0), 10),
                   (B(_abi.BSA_BUDGET_TOPK, 4, 0, 0, 0, 0.0), 0)]:
        assert L.bsa_select_max_count(ctypes.byref(bad), n) == _abi.BSA_ERR_INVALID_ARG
        assert L.bsa_last_error()
    assert L.bsa_select_max_count(None, 10) == _abi.BSA_ERR_INVALID_ARG


def test_select_argument_checks():
    kv = _kv()
    B = _abi.bsa_budget
    assert _select(kv, B(_abi.BSA_BUDGET_TOPK, 0, 0, 0, 0, 0.0), 8) == _abi.BSA_ERR_INVALID_ARG
    assert _select(kv, B(_abi.BSA_BUDGET_TOPK, 16, 0, 0, 0, 0.0), 8) == _abi.BSA_ERR_INVALID_ARG  # max_sel < 16
    assert _select(kv, B(_abi.BSA_BUDGET_RATIO, 0, 0, 1, 1, 0.0), 64) == _abi.BSA_ERR_INVALID_ARG
    assert _select(kv, B(_abi.BSA_BUDGET_RATIO, 0, 0, 2, 1, 0.5), 64) == _abi.BSA_ERR_INVALID_ARG
    # ratio 0.5 over 64 pages -> 32 kept; max_sel 31 is too small
    assert _select(kv, B(_abi.BSA_BUDGET_RATIO, 0, 0, 1, 1, 0.5), 31) == _abi.BSA_ERR_INVALID_ARG
    assert _select(kv, B(_abi.BSA_BUDGET_TOKENS, 0, 0, 0, 0, 0.0), 8) == _abi.BSA_ERR_INVALID_ARG
    assert _select(kv, B(9, 1, 0, 0, 0, 0.0), 8) == _abi.BSA_ERR_INVALID_ARG
    assert _select(_kv(max_pages=16385), B(_abi.BSA_BUDGET_TOPK, 4, 0, 0, 0, 0.0), 8) == _abi.BSA_ERR_UNSUPPORTED
    ch = _abi.bsa_chunks(FAKE, None, 10)
    assert _select(kv, B(_abi.BSA_BUDGET_TOPK, 4, 0, 0, 0, 0.0), 8, ctypes.byref(ch)) == _abi.BSA_ERR_INVALID_ARG


def test_router_argument_checks():
    L = _abi.lib()

    def call(nt=8, H=2, nb=8, k=2, rho=2, quant=0.25, fixed=float("nan"), ws=FAKE, wsb=1 << 20):
        return L.bsa_select_topk_router(FAKE, nt, H, nb, 1, k, rho, quant, fixed, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                                        wsb, None)

    assert L.bsa_router_workspace_bytes(2048, 4, 32, 2) == 0     # no scratch: lists go straight to kv_idx
    assert call(k=200, rho=2) == _abi.BSA_ERR_UNSUPPORTED
    assert call(k=256, rho=1) == _abi.BSA_ERR_UNSUPPORTED        # needs k+1 = 257 sorted scores
    assert call(nb=9000) == _abi.BSA_ERR_UNSUPPORTED
    assert call(nt=9000) == _abi.BSA_ERR_UNSUPPORTED
    assert call(quant=1.5) == _abi.BSA_ERR_INVALID_ARG
    assert call(k=0) == _abi.BSA_ERR_INVALID_ARG


def test_meta_and_score_argument_checks():
    L = _abi.lib()
    kv = _kv()
    m = _abi.bsa_meta(FAKE, None, None)
    assert L.bsa_build_chunk_meta(ctypes.byref(kv), None, ctypes.byref(m), _abi.BSA_META_ENVELOPE,
                                  None) == _abi.BSA_ERR_INVALID_ARG
    assert L.bsa_build_chunk_meta(ctypes.byref(kv), None, ctypes.byref(m), 0, None) == _abi.BSA_ERR_INVALID_ARG
    assert L.bsa_build_chunk_meta(ctypes.byref(kv), None, None, 1, None) == _abi.BSA_ERR_INVALID_ARG
    m2 = _abi.bsa_meta(FAKE, FAKE, None)
    # centroid scoring without a centroid buffer
    assert L.bsa_score_chunks(FAKE, 8, 1, 1, ctypes.byref(kv), None, ctypes.byref(m2), _abi.BSA_CENTROID, 0,
                              FAKE, None) == _abi.BSA_ERR_INVALID_ARG
    # decode scoring needs num_rows == batch
    assert L.bsa_score_chunks(FAKE, 8, 3, 1, ctypes.byref(kv), None, ctypes.byref(m2), _abi.BSA_ENVELOPE, 0,
                              FAKE, None) == _abi.BSA_ERR_INVALID_ARG
    # tile scoring: 64-row tiles over 64-token blocks only
    assert L.bsa_score_chunks(FAKE, 8, 128, 32, ctypes.byref(kv), None, ctypes.byref(m2), _abi.BSA_ENVELOPE, 1,
                              FAKE, None) == _abi.BSA_ERR_UNSUPPORTED
    kvt = _kv(page_size=64, stride_page=64 * 2 * 128, stride_head=128, stride_token=256, block_table=None)
    assert L.bsa_score_chunks(FAKE, 18, 128, 64, ctypes.byref(kvt), None, ctypes.byref(m2), _abi.BSA_ENVELOPE, 1,
                              FAKE, None) == _abi.BSA_ERR_UNSUPPORTED   # group 9 > 8


def test_tile_prefill_argument_checks():
    L = _abi.lib()
    kvt = _kv(page_size=64, stride_page=64 * 2 * 128, stride_head=128, stride_token=256, block_table=None)
    need = L.bsa_tile_prefill_workspace_bytes(ctypes.byref(kvt), 256)
    assert need == 256 * 2 * 128 * 2                                    # fp16 V [rows][H_kv][D]
    call = lambda kv, hq=8, tile=64, stride=4, idx=FAKE, ws=FAKE, wsb=need: L.bsa_sparse_attn_tile_prefill(
        FAKE, hq, 256, ctypes.byref(kv), tile, idx, stride, 0.088, FAKE, ws, wsb, None)
    assert call(kvt, ws=None) == _abi.BSA_ERR_WORKSPACE
    assert call(kvt, wsb=need - 1) == _abi.BSA_ERR_WORKSPACE
    assert call(kvt, ws=FAKE + 8) == _abi.BSA_ERR_INVALID_ARG          # alignment
    assert call(_kv()) == _abi.BSA_ERR_UNSUPPORTED                    # paged with a block table
    assert call(kvt, tile=32) == _abi.BSA_ERR_UNSUPPORTED
    assert call(kvt, hq=18) == _abi.BSA_ERR_UNSUPPORTED
    assert call(kvt, stride=0) == _abi.BSA_ERR_INVALID_ARG
    assert call(kvt, stride=1025) == _abi.BSA_ERR_UNSUPPORTED
    assert call(_kv(page_size=64, stride_page=64 * 2 * 128, stride_head=128, stride_token=256, block_table=None,
                    dtype=_abi.BSA_F32, head_dim=128)) == _abi.BSA_ERR_UNSUPPORTED


def test_fused_select_decode_argument_checks():
    L = _abi.lib()
    B = _abi.bsa_budget
    top = B(_abi.BSA_BUDGET_TOPK, 8, 0, 0, 0, 0.0)

    def call(kv=None, hq=8, budget=top, splits=0, sel=False, cnt=False, max_sel=0, ws=None, wsb=0, scale=0.088):
        kv = kv or _kv()
        return L.bsa_select_attn_decode(FAKE, hq, ctypes.byref(kv), FAKE, ctypes.byref(budget), scale, splits, FAKE,
                                        FAKE if sel else None, FAKE if cnt else None, max_sel, ws, wsb, None)

    assert call(kv=_kv(page_size=32)) == _abi.BSA_ERR_UNSUPPORTED
    assert call(kv=_kv(max_pages=16385)) == _abi.BSA_ERR_UNSUPPORTED
    # rows of more than 8192 pages: the selection kernel, then the split-grid
    # attention; the kept lists (top-8: 8 + the count per row) follow the
    # partials in the workspace unless sel_idx is given
    long = _kv(max_pages=9000)
    s9 = L.bsa_decode_num_splits(ctypes.byref(long), 8, 8, 0)
    part = 1 * 8 * s9 * 130 * 4 if s9 > 1 else 0
    lists = 1 * 2 * (8 + 1) * 4
    need9 = L.bsa_decode_workspace_bytes(ctypes.byref(long), 8, 8, 0)
    assert need9 == ((part + 15) & ~15) + lists
    assert call(kv=long) == _abi.BSA_ERR_WORKSPACE
    assert call(kv=long, ws=FAKE, wsb=need9 - 1) == _abi.BSA_ERR_WORKSPACE
    assert call(hq=34) == _abi.BSA_ERR_UNSUPPORTED
    assert call(sel=True) == _abi.BSA_ERR_INVALID_ARG                    # sel_idx without sel_count
    assert call(sel=True, cnt=True, max_sel=7) == _abi.BSA_ERR_INVALID_ARG  # 8 pages may be kept
    assert call(splits=65) == _abi.BSA_ERR_INVALID_ARG
    assert call(scale=-1.0) == _abi.BSA_ERR_INVALID_ARG
    assert call(budget=B(_abi.BSA_BUDGET_RATIO, 0, 0, 1, 1, 0.0)) == _abi.BSA_ERR_INVALID_ARG
    # 4096 pages in one split exceed the 2048 kept per split
    big = _kv(max_pages=4096)
    assert call(kv=big, budget=B(_abi.BSA_BUDGET_TOPK, 4096, 0, 0, 0, 0.0), splits=1) == _abi.BSA_ERR_INVALID_ARG
    assert "splits" in L.bsa_last_error().decode()
    # automatic splits respect that limit
    assert L.bsa_decode_num_splits(ctypes.byref(_kv(batch=64, num_kv_heads=8, max_pages=8192)), 64, 8192, 0) >= 4
    need = L.bsa_decode_workspace_bytes(ctypes.byref(_kv()), 8, 8, 4)
    assert need == 1 * 8 * 4 * 130 * 4
    assert call(splits=4) == _abi.BSA_ERR_WORKSPACE
    assert call(splits=4, ws=FAKE, wsb=need - 1) == _abi.BSA_ERR_WORKSPACE


def test_merge_and_partials_argument_checks():
    L = _abi.lib()
    assert L.bsa_decode_merge(None, 1, 8, 128, 4, FAKE, None) == _abi.BSA_ERR_INVALID_ARG
    assert L.bsa_decode_merge(FAKE, 1, 8, 96, 4, FAKE, None) == _abi.BSA_ERR_UNSUPPORTED
    assert L.bsa_decode_merge(FAKE, 1, 8, 128, 1, FAKE, None) == _abi.BSA_ERR_INVALID_ARG
    assert L.bsa_decode_merge(FAKE, 1, 8, 128, 65, FAKE, None) == _abi.BSA_ERR_INVALID_ARG
    assert L.bsa_decode_merge(FAKE, 0, 8, 128, 4, FAKE, None) == _abi.BSA_ERR_INVALID_ARG
    # out == NULL needs more than one split
    kv = _kv()
    rc = L.bsa_sparse_attn_decode(FAKE, 8, ctypes.byref(kv), None, FAKE, FAKE, 8, 0.088, 1, None, None, 0, None)
    assert rc == _abi.BSA_ERR_INVALID_ARG and "out may be NULL" in L.bsa_last_error().decode()


def test_update_meta_argument_checks():
    L = _abi.lib()
    kv = _kv()
    m = _abi.bsa_meta(FAKE, FAKE, FAKE)
    def upd(mt, which=3, meta=ctypes.byref(m)):
        return L.bsa_update_chunk_meta(ctypes.byref(kv), None, meta, which, None, mt, None)
    assert upd(0) == _abi.BSA_ERR_INVALID_ARG
    assert upd(65) == _abi.BSA_ERR_INVALID_ARG                # max_pages is 64
    assert upd(1, which=0) == _abi.BSA_ERR_INVALID_ARG
    assert upd(1, meta=None) == _abi.BSA_ERR_INVALID_ARG
    assert "max_touched" in (upd(0) and L.bsa_last_error().decode())


def test_meta_arrays_must_be_16_byte_aligned():
    L = _abi.lib()
    kv = _kv()
    for bad in (_abi.bsa_meta(FAKE + 2, FAKE, FAKE), _abi.bsa_meta(FAKE, FAKE + 8, FAKE),
                _abi.bsa_meta(FAKE, FAKE, FAKE + 4)):
        assert L.bsa_build_chunk_meta(ctypes.byref(kv), None, ctypes.byref(bad), 3, None) == _abi.BSA_ERR_INVALID_ARG
        assert "16-byte aligned" in L.bsa_last_error().decode()
        assert L.bsa_update_chunk_meta(ctypes.byref(kv), None, ctypes.byref(bad), 3, None, 1,
                                       None) == _abi.BSA_ERR_INVALID_ARG
        rc = L.bsa_score_chunks(FAKE, 8, 1, 1, ctypes.byref(kv), None, ctypes.byref(bad), _abi.BSA_ENVELOPE, 0,
                                FAKE, None)
        assert rc == _abi.BSA_ERR_INVALID_ARG and "16-byte aligned" in L.bsa_last_error().decode()


def test_decode_outputs_must_be_16_byte_aligned():
    L = _abi.lib()
    kv = _kv()
    need = L.bsa_decode_workspace_bytes(ctypes.byref(kv), 8, 8, 4)
    # unfused decode: out, then workspace
    rc = L.bsa_sparse_attn_decode(FAKE, 8, ctypes.byref(kv), None, FAKE, FAKE, 8, 0.088, 1, FAKE + 8, None, 0, None)
    assert rc == _abi.BSA_ERR_INVALID_ARG and "out must be 16-byte aligned" in L.bsa_last_error().decode()
    rc = L.bsa_sparse_attn_decode(FAKE, 8, ctypes.byref(kv), None, FAKE, FAKE, 8, 0.088, 4, FAKE, FAKE + 4, need, None)
    assert rc == _abi.BSA_ERR_INVALID_ARG and "workspace must be 16-byte aligned" in L.bsa_last_error().decode()
    # fused selection + decode
    top = _abi.bsa_budget(_abi.BSA_BUDGET_TOPK, 8, 0, 0, 0, 0.0)
    rc = L.bsa_select_attn_decode(FAKE, 8, ctypes.byref(kv), FAKE, ctypes.byref(top), 0.088, 4, FAKE + 4,
                                  None, None, 0, FAKE, need, None)
    assert rc == _abi.BSA_ERR_INVALID_ARG and "out must be 16-byte aligned" in L.bsa_last_error().decode()
    rc = L.bsa_select_attn_decode(FAKE, 8, ctypes.byref(kv), FAKE, ctypes.byref(top), 0.088, 4, FAKE,
                                  None, None, 0, FAKE + 8, need, None)
    assert rc == _abi.BSA_ERR_INVALID_ARG and "workspace" in L.bsa_last_error().decode()
    # merge
    assert L.bsa_decode_merge(FAKE + 4, 1, 8, 128, 4, FAKE, None) == _abi.BSA_ERR_INVALID_ARG
    assert L.bsa_decode_merge(FAKE, 1, 8, 128, 4, FAKE + 8, None) == _abi.BSA_ERR_INVALID_ARG


def test_static_scratch_entry_point_refuses_before_any_hip_call():
    """bsa_select_attn_decode_static checks its arguments and its scratch need
    on the host: out NULL and a plan needing more than the static scratch are
    refused without a device."""
    L = _abi.lib()
    top = _abi.bsa_budget(_abi.BSA_BUDGET_TOPK, 8, 0, 0, 0, 0.0)

    def call(kv, hq, budget=top, out=FAKE):
        return L.bsa_select_attn_decode_static(FAKE, hq, ctypes.byref(kv), FAKE, ctypes.byref(budget), 0.088, 0,
                                               out, None, None, 0, None)

    assert call(_kv(), 8, out=None) == _abi.BSA_ERR_INVALID_ARG
    assert "out" in L.bsa_last_error().decode()
    assert call(_kv(page_size=32, stride_page=2 * 32 * 128, stride_head=32 * 128), 8) == _abi.BSA_ERR_UNSUPPORTED
    # 4096 rows, groups of 16 heads, balanced schedule: (4096 + 256) x 16 x 130
    # floats of partials alone exceed 16 MiB
    big = _kv(batch=4096, num_kv_heads=1, max_pages=64)
    top64 = _abi.bsa_budget(_abi.BSA_BUDGET_TOPK, 64, 0, 0, 0, 0.0)
    need = L.bsa_decode_workspace_bytes(ctypes.byref(big), 16, 64, 0)
    assert need > _abi.BSA_STATIC_SCRATCH_BYTES
    assert call(big, 16, budget=top64) == _abi.BSA_ERR_UNSUPPORTED
    msg = L.bsa_last_error().decode()
    assert str(need) in msg and str(_abi.BSA_STATIC_SCRATCH_BYTES) in msg


def test_ceiling_library_refuses_bad_arguments_before_any_hip_call():
    """libbsa_ceiling.so (the benchmark's gather-ceiling kernel) exports its one
    entry point and rejects missing buffers, empty run lists and a zero share
    per wave on the host (hipErrorInvalidValue = 1), before any HIP call."""
    path = os.path.join(os.path.dirname(_abi.LIB_PATH), "libbsa_ceiling.so")
    if not os.path.exists(path):
        pytest.skip("libbsa_ceiling.so not built")
    lib = ctypes.CDLL(path)
    f = lib.bsa_ceiling_gather
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    buf = ctypes.create_string_buffer(64)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert f(None, p, 4, 1, p, None) == 1
    assert f(p, None, 4, 1, p, None) == 1
    assert f(p, p, 4, 1, None, None) == 1
    assert f(p, p, 0, 1, p, None) == 1
    assert f(p, p, 4, 0, p, None) == 1
