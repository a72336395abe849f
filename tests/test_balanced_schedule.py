"""Host-side check of the balanced decode schedule's bookkeeping (no GPU).

The attention kernel lays the rows' kept pages end to end (row r holds
positions [P_r, P_r + n_r)), gives workgroup w the positions
[w qn, (w + 1) qn) with qn = max(ceil(T / 256), 16), and stores the partial
of (row r, workgroup w) at entry r + w; the merge reads, for row r, the entries
r + w for w from P_r // qn to (P_r + n_r - 1) // qn.  This file enumerates the
segments the way the kernel does and checks, over many random count vectors
(empty rows, single pages, one dominant row), that no two segments share an
entry, that every entry stays below rows + 256 (the workspace size), that the
merge's entry range of each row is exactly the set of its segments, and that
the segments of a row cover its positions once.
"""
import numpy as np
import pytest

WGS, MIN_ITEMS = 256, 16


def segments(counts):
    counts = np.asarray(counts, dtype=np.int64)
    rows = len(counts)
    pre = np.concatenate([[0], np.cumsum(counts)])
    total = int(pre[-1])
    qn = max(-(-total // WGS), MIN_ITEMS)
    segs = []                                   # (row, workgroup, first item, end item)
    for w in range(WGS):
        start = w * qn
        if start >= total:
            break
        end = min(start + qn, total)
        r = int(np.searchsorted(pre[1:], start, side="right"))   # the row holding `start`
        while r < rows and pre[r] < end:
            a, e = max(start, pre[r]) - pre[r], min(end, pre[r + 1]) - pre[r]
            if e > a:
                segs.append((r, w, int(a), int(e)))
            r += 1
    return segs, pre, qn


def merge_entries(r, pre, qn, counts):
    n = int(counts[r])
    if n == 0:
        return []
    w0, w1 = int(pre[r]) // qn, (int(pre[r]) + n - 1) // qn
    return [r + w for w in range(w0, w1 + 1)]


@pytest.mark.parametrize("seed", range(40))
def test_entries_unique_bounded_and_matching_the_merge(seed):
    gen = np.random.default_rng(seed)
    rows = int(gen.integers(16, 300))
    kind = seed % 4
    if kind == 0:
        counts = gen.integers(0, 2000, size=rows)
    elif kind == 1:
        counts = gen.integers(0, 3, size=rows)                  # tiny and empty rows
    elif kind == 2:
        counts = np.zeros(rows, dtype=np.int64)
        counts[gen.integers(rows)] = int(gen.integers(1, 8192))  # one dominant row
        counts[gen.integers(rows, size=5)] += 1
    else:
        counts = np.full(rows, int(gen.integers(1, 600)))        # equal rows
    segs, pre, qn = segments(counts)
    entries = [r + w for r, w, _, _ in segs]
    assert len(entries) == len(set(entries))
    assert all(0 <= e < rows + WGS for e in entries)
    by_row = {}
    for r, w, a, e in segs:
        by_row.setdefault(r, []).append((w, a, e))
    for r in range(rows):
        got = sorted(by_row.get(r, []))
        assert [r + w for w, _, _ in got] == merge_entries(r, pre, qn, counts)
        # the row's items are covered once, in order
        pos = 0
        for _, a, e in got:
            assert a == pos
            pos = e
        assert pos == counts[r]
