"""The balanced partition of paged_decode_attn (num_splits = -W), stated on
the host and checked on random batches: per KV head, the live requests'
pages in request order form one sequence of T pages, and work-group w takes
pages [w C, min((w + 1) C, T)) with C = ceil(T / W).  A piece (request b,
work-group w) is written whole when the request lies inside the range, else
as a partial at row b + w of its query head; the combine recovers a request's
rows from its first page in the sequence and C.  The checks: every live page
is covered exactly once, no two pieces share a row, rows stay inside the
B + W - 1 the workspace holds, and the combine's rows are exactly the
pieces'.  This is the integer bookkeeping only; the arithmetic is covered by
the GPU parity tests."""
import numpy as np
import pytest

from paged_attention_fp8_amd import ops


def pages_of(L, status, P, max_pages):
    """Pages a request adds to the sequence (0 for aborted, empty, invalid)."""
    if status != 0 or L <= 0 or L > max_pages * P:
        return 0
    return -(-L // P)


def partition(lens, status, P, max_pages, W):
    n = [pages_of(int(L), int(s), P, max_pages) for L, s in zip(lens, status)]
    prefix = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
    T = int(prefix[-1])
    C = -(-T // W) if T > 0 else 1
    pieces = []   # (b, w, first page, end page, whole)
    for w in range(W):
        lo, hi = w * C, min(w * C + C, T)
        if lo >= hi:
            continue
        b = int(np.searchsorted(prefix, lo, side="right")) - 1
        while b < len(n) and n[b] == 0:
            b += 1
        ps = int(prefix[b])
        while b < len(n) and ps < hi:
            if n[b] > 0:
                p0, p1 = max(lo, ps) - ps, min(hi, ps + n[b]) - ps
                whole = ps >= lo and ps + n[b] <= hi
                pieces.append((b, w, p0, p1, whole))
            ps += n[b]
            b += 1
    return n, prefix, C, pieces


@pytest.mark.parametrize("seed", range(40))
def test_pieces_cover_rows_unique_and_combine_agrees(seed):
    g = np.random.default_rng(seed)
    B = int(g.integers(1, 40))
    P = int(g.choice([16, 64, 256]))
    max_pages = int(g.integers(1, 64))
    lens = g.integers(0, max_pages * P + 1, B)
    if g.random() < 0.5:
        lens[g.random(B) < 0.2] = 0
    if g.random() < 0.3:
        lens[g.integers(0, B)] = max_pages * P + 1      # invalid: past the table
    status = np.where(g.random(B) < 0.1, 2, 0)
    W = int(g.choice([1, 2, 3, 7, 32, 200]))
    n, prefix, C, pieces = partition(lens, status, P, max_pages, W)
    R = B + W - 1
    # every live page exactly once
    cover = [np.zeros(k, np.int32) for k in n]
    for b, w, p0, p1, _ in pieces:
        assert 0 <= p0 < p1 <= n[b]
        cover[b][p0:p1] += 1
    assert all(np.all(c == 1) for c in cover)
    # partial rows unique and in range
    rows = [b + w for b, w, _, _, whole in pieces if not whole]
    assert len(rows) == len(set(rows))
    assert all(0 <= r < R for r in rows)
    # the combine's view: rows b + w0 .. b + w1, or written whole when w0 == w1
    for b in range(B):
        mine = sorted((w, whole) for bb, w, _, _, whole in pieces if bb == b)
        if n[b] == 0:
            assert not mine
            continue
        w0, w1 = int(prefix[b]) // C, (int(prefix[b]) + n[b] - 1) // C
        assert [w for w, _ in mine] == list(range(w0, w1 + 1))
        assert all(whole == (w0 == w1) for _, whole in mine)
    # each work-group's range holds at most C pages
    per_w = {}
    for b, w, p0, p1, _ in pieces:
        per_w[w] = per_w.get(w, 0) + p1 - p0
    assert all(v <= C for v in per_w.values())


def test_workspace_size_formula():
    B, Hq, D = 32, 64, 128
    for W in (1, 32, 65536):
        R = B + W - 1
        want = (-(-Hq * R * D * 4 // 16) * 16) + (-(-Hq * R * 4 // 16) * 16) + (B + 1) * 8
        assert ops.workspace_bytes(B, Hq, D, -W) == want
    assert ops.workspace_bytes(B, Hq, D, -65537) == 0     # out of range: rejected by the call
    assert ops.default_balanced_groups(8, 256) == 32
    assert ops.default_balanced_groups(3, 256) == 86
    assert ops.default_balanced_groups(1024, 256) == 1
