"""Pins for the oracle's page-tag check (O6), pool writes (O4/O5) and combine
(O8), and for the host page pool.

The check follows the shared-cache protection section of Cloudflare's
"Smaller, faster, safer: running Kimi and GLM at scale" ("共享 KV 缓存保护"):
each physical page has a tag that changes on reallocation, each request
records the pages and tags it expects, the mapping is verified before decode
reads, and a mismatching request is terminated.  Its expected outcome is known
by construction from host-side injection, and a plain Python brute force
recomputes it.  The capacity invariants follow the KV cache quantization
section ("KV 缓存量化"): e4m3 halves the cache, so the same memory holds twice
the tokens, and the bf16 cache refuses the 33rd request where e4m3 reaches 64.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from paged_attention_fp8_amd import inputs as I
from helpers import oracle_pool


def _brute_status(table, lens, expected, tags, P):
    out = []
    for b in range(len(lens)):
        L = int(lens[b])
        if L < 1 or L > table.shape[1] * P:
            out.append(oracle.REQ_BAD_LEN)
            continue
        st = 0
        for i in range(-(-L // P)):
            p = int(table[b, i])
            if not 0 <= p < len(tags):
                st |= oracle.REQ_PAGE_OOB
            elif int(tags[p]) != int(expected[b, i]):
                st |= oracle.REQ_TAG_MISMATCH
        out.append(st)
    return np.array(out, np.int32)


def test_tag_check_clean_batch_all_ok():
    pool = I.PagePool(400, seed=1)
    batch = I.allocate_batch(pool, [1, 16, 17, 100, 333], 16)
    st = oracle.page_tag_check(batch.page_table, batch.context_lens, batch.expected_tags,
                               pool.tags, 16)
    assert np.all(st == 0)


def test_tag_check_stale_oob_badlen_by_construction():
    P = 16
    pool = I.PagePool(1000, seed=2)
    lens = np.array([40, 200, 16, 1, 500, 77, 300, 64], np.int32)
    batch = I.allocate_batch(pool, lens, P)
    I.make_stale(pool, batch, 1, 5)               # request 1: stale page
    I.make_stale(pool, batch, 6, 0)               # request 6: stale first page
    batch.page_table[3, 0] = 1000                 # request 3: page id beyond the pool
    batch.page_table[4, 2] = -7                   # request 4: negative page id
    I.make_stale(pool, batch, 4, 3)               #   ... and a stale page
    lens2 = lens.copy()
    lens2[5] = 0                                  # request 5: empty
    lens2[7] = batch.max_pages * P + 1            # request 7: longer than its table
    st = oracle.page_tag_check(batch.page_table, lens2, batch.expected_tags, pool.tags, P)
    want = np.zeros(8, np.int32)
    want[1] = want[6] = oracle.REQ_TAG_MISMATCH
    want[3] = oracle.REQ_PAGE_OOB
    want[4] = oracle.REQ_PAGE_OOB | oracle.REQ_TAG_MISMATCH
    want[5] = want[7] = oracle.REQ_BAD_LEN
    assert np.array_equal(st, want)
    assert np.array_equal(st, _brute_status(batch.page_table, lens2, batch.expected_tags,
                                            pool.tags, P))


def test_tag_check_only_pages_in_use_are_checked():
    # a stale tag on a page slot beyond the context is not the request's concern
    P = 16
    pool = I.PagePool(64, seed=3)
    batch = I.allocate_batch(pool, [48], P, max_pages=4)
    batch.page_table[0, 3] = 5
    batch.expected_tags[0, 3] = 12345
    st = oracle.page_tag_check(batch.page_table, batch.context_lens, batch.expected_tags,
                               pool.tags, P)
    assert st[0] == 0


def test_tag_check_random_vs_brute():
    g = np.random.default_rng(4)
    for trial in range(20):
        P = int(g.choice([16, 32, 64]))
        B = int(g.integers(1, 40))
        pool = I.PagePool(int(g.integers(200, 2000)), seed=trial)
        lens = g.integers(1, 20 * P, B)
        try:
            batch = I.allocate_batch(pool, lens, P)
        except I.PoolExhausted:
            continue
        for _ in range(int(g.integers(0, 5))):
            b = int(g.integers(0, B))
            I.make_stale(pool, batch, b, int(g.integers(0, I.pages_needed(lens[b], P))))
        lens = lens.astype(np.int32)
        lens[g.random(B) < 0.1] = 0
        st = oracle.page_tag_check(batch.page_table, lens, batch.expected_tags, pool.tags, P)
        assert np.array_equal(st, _brute_status(batch.page_table, lens, batch.expected_tags,
                                                pool.tags, P))


def test_tag_check_thousand_requests_one_stale():
    """0.1% of 1000 requests (one) carries a stale tag: exactly it is flagged."""
    P = 64
    pool = I.PagePool(1000 * 64 + 10, seed=5)
    batch = I.allocate_batch(pool, np.full(1000, 64 * 64, np.int32), P)
    I.make_stale(pool, batch, 437, 17)
    st = oracle.page_tag_check(batch.page_table, batch.context_lens, batch.expected_tags,
                               pool.tags, P)
    assert np.flatnonzero(st).tolist() == [437] and st[437] == oracle.REQ_TAG_MISMATCH


# --- O6b: reallocation ---------------------------------------------------------------

def test_realloc_reproduces_the_host_allocator():
    """Replaying the host allocator's allocations as reallocation entries gives
    its tags, page table and recorded tags (two independent implementations
    of 'every allocation moves the page's tag on')."""
    pool = I.PagePool(300, seed=5, first_tag=7)
    tags0 = pool.tags.copy()
    batch = I.allocate_batch(pool, [40, 900, 1, 513, 64], 16)
    ids, reqs, slots = [], [], []
    for b in range(batch.batch):
        n = I.pages_needed(batch.context_lens[b], 16)
        ids += list(batch.page_table[b, :n])
        reqs += [b] * n
        slots += list(range(n))
    table0 = np.full_like(batch.page_table, -1)
    exp0 = np.zeros_like(batch.expected_tags)
    tags, table, exp = oracle.page_tag_realloc(ids, tags0, reqs, slots, table0, exp0)
    assert np.array_equal(tags, pool.tags)
    assert np.array_equal(table, batch.page_table)
    assert np.array_equal(exp, batch.expected_tags)


def test_realloc_makes_the_old_owner_stale_and_the_new_one_valid():
    """A page given to another request: the old holder fails the check with a
    tag mismatch, the new holder passes, everyone else is unchanged."""
    pool = I.PagePool(64, seed=1)
    batch = I.allocate_batch(pool, [48, 48, 48], 16)   # 3 pages each
    check = lambda t, tb, e: oracle.page_tag_check(tb, batch.context_lens, e, t, 16)
    assert np.all(check(pool.tags, batch.page_table, batch.expected_tags) == 0)
    victim = int(batch.page_table[0, 1])
    # request 2 takes over the page as its logical page 2
    tags, table, exp = oracle.page_tag_realloc([victim], pool.tags, [2], [2], batch.page_table,
                                               batch.expected_tags)
    st = check(tags, table, exp)
    assert list(st) == [oracle.REQ_TAG_MISMATCH, 0, 0]
    assert table[2, 2] == victim and exp[2, 2] == pool.tags[victim] + 1


def test_realloc_edges():
    tags0 = np.array([0xFFFFFFFF, 5, 9], np.uint32)
    # wrap-around, out-of-pool entries, owners outside the table
    tags, table, exp = oracle.page_tag_realloc([0, 3, -1, 1], tags0, [0, 0, 0, 7], [1, 0, 0, 0],
                                               np.full((2, 2), -1, np.int32), np.zeros((2, 2), np.uint32))
    assert list(tags) == [0, 6, 9]
    assert table[0, 1] == 0 and exp[0, 1] == 0          # the wrapped tag is recorded
    assert np.count_nonzero(table != -1) == 1             # page 3 and -1 are outside; owner 7 too
    # without owners only the tags move; a page listed twice moves twice
    tags, table, exp = oracle.page_tag_realloc([2, 2, 1], tags0)
    assert list(tags) == [0xFFFFFFFF, 6, 11] and table is None and exp is None


# --- pool writes -----------------------------------------------------------------

def test_block_layout_maps_are_permutations():
    from helpers import block_index_maps
    for kv in (oracle.KV_FP8, oracle.KV_BF16):
        for P in (16, 32, 64, 128, 256):
            for D in (64, 128):
                kmap, vmap = block_index_maps(kv, P, D)
                assert np.array_equal(np.sort(kmap.ravel()), np.arange(P * D))
                assert np.array_equal(np.sort(vmap.ravel()), np.arange(P * D))


def test_block_layout_shape_properties():
    """The properties the layout exists for: a segment is one wave tile (64
    e4m3 / 32 bf16 tokens) when the page holds it; each 16-byte load step of
    a tile's K (the 64 lanes' chunks) is one contiguous kilobyte; a V row of
    the segment is contiguous."""
    from helpers import block_index_maps
    for kv, TT, TG in ((oracle.KV_FP8, 64, 16), (oracle.KV_BF16, 32, 8)):
        kmap, vmap = block_index_maps(kv, 128, 128)
        e = 1 if kv == oracle.KV_FP8 else 2
        KL = 128 * e // 64
        for j in range(TG // 4):
            for l in range(KL):
                # lane (q, r) reads chunk q*KL + l of token TG*(r//4) + 4j + r%4
                pos = sorted(int(kmap[TG * (r // 4) + 4 * j + r % 4, (q * KL + l) * 16 // e]) * e
                             for q in range(4) for r in range(16))
                assert pos == list(range(pos[0], pos[0] + 1024, 16))
        assert np.array_equal(vmap[:TT, 5], vmap[0, 5] + np.arange(TT))
        assert vmap[TT, 0] == 128 * TT  # the next segment starts after D rows


def test_oracle_offsets_match_documented_layout():
    from helpers import block_index_maps
    g = np.random.default_rng(9)
    for kv in (oracle.KV_FP8, oracle.KV_BF16):
        for P, D, Hkv in ((16, 64, 3), (64, 128, 2), (256, 128, 1), (32, 64, 4)):
            kmap, vmap = block_index_maps(kv, P, D)
            for _ in range(200):
                page, h = int(g.integers(0, 50)), int(g.integers(0, Hkv))
                t, d = int(g.integers(0, P)), int(g.integers(0, D))
                base = (page * Hkv + h) * P * D
                assert oracle.k_offset(kv, page, h, t, d, Hkv, P, D) == base + kmap[t, d]
                assert oracle.v_offset(kv, page, h, t, d, Hkv, P, D) == base + vmap[t, d]


def test_pool_write_layout_and_codes():
    """Tokens written through the oracle land at the documented positions, as
    torch's e4m3 encoding of f32(x)/scale."""
    from helpers import kv_rows
    w = I.Workload("w", 2, 4, 2, 64, 16, 19, 40, pool_factor=2.0)
    inp = I.make_decode_inputs(w, 3)
    pool = oracle_pool(inp, oracle.KV_FP8, poison=False)
    enc = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for b in range(2):
        L = int(inp.batch.context_lens[b])
        t = np.arange(L)
        pages = inp.batch.page_table[b][t // w.page_size]
        kc, vc = kv_rows(pool, pages, t % w.page_size)
        x_k = I.bf16_bits_to_f32(inp.k_tokens[b]) / inp.k_scale[None, :, None]
        x_v = I.bf16_bits_to_f32(inp.v_tokens[b]) / inp.v_scale[None, :, None]
        assert np.array_equal(kc, enc(x_k))
        assert np.array_equal(vc, enc(x_v))


def test_append_equals_bulk_write_of_last_token():
    w = I.Workload("w", 3, 4, 2, 64, 16, 5, 40, pool_factor=2.0)
    inp = I.make_decode_inputs(w, 4)
    a = oracle_pool(inp, oracle.KV_FP8, poison=False, append=True)
    b = oracle_pool(inp, oracle.KV_FP8, poison=False, append=False)
    lens = inp.batch.context_lens
    oracle.kv_write(b, inp.batch.page_table, lens - 1, np.ones(3, np.int32),
                    inp.k_new()[:, None], inp.v_new()[:, None], inp.k_scale, inp.v_scale)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)


def test_append_skips_aborted_and_invalid():
    w = I.Workload("w", 3, 4, 2, 64, 16, 20, 20, pool_factor=2.0)
    inp = I.make_decode_inputs(w, 5)
    base = oracle_pool(inp, oracle.KV_FP8, poison=False, append=False)
    k0, v0 = base.k.copy(), base.v.copy()
    lens = inp.batch.context_lens.copy()
    lens[2] = 0
    oracle.kv_append(base, inp.batch.page_table, lens, inp.k_new(), inp.v_new(), inp.k_scale,
                     inp.v_scale, status=np.array([0, 1, 0], np.int32))
    changed = np.argwhere(base.k != k0)
    pages_changed = set(int(p) for p in changed[:, 0])
    assert pages_changed == {int(inp.batch.page_table[0, 19 // 16])}
    assert (base.v != v0).any()


def test_bf16_append_copies_bits():
    from helpers import kv_rows
    w = I.Workload("w", 2, 2, 2, 64, 16, 3, 9, pool_factor=2.0)
    inp = I.make_decode_inputs(w, 6)
    pool = oracle_pool(inp, oracle.KV_BF16, poison=False)
    for b in range(2):
        t = int(inp.batch.context_lens[b]) - 1
        page, slot = inp.batch.page_table[b, t // 16], t % 16
        kc, vc = kv_rows(pool, [page], [slot])
        assert np.array_equal(kc[0], inp.k_new()[b])
        assert np.array_equal(vc[0], inp.v_new()[b])


# --- capacity invariants ---------------------------------------------------------

def test_fp8_cache_is_exactly_half_of_bf16():
    a = oracle.Pool(oracle.KV_FP8, 37, 8, 64, 128)
    b = oracle.Pool(oracle.KV_BF16, 37, 8, 64, 128)
    assert 2 * (a.k.nbytes + a.v.nbytes) == b.k.nbytes + b.v.nbytes


def test_same_budget_holds_64_fp8_or_32_bf16_requests():
    n8 = I.pages_in_budget(I.SWEEP_BUDGET_BYTES, 8, 64, 128, 1)
    n16 = I.pages_in_budget(I.SWEEP_BUDGET_BYTES, 8, 64, 128, 2)
    assert n8 == 2 * n16 == 16384
    fp8 = I.PagePool(n8, seed=0)
    I.allocate_batch(fp8, [16384] * 64, 64)
    assert fp8.free_pages == 0
    bf = I.PagePool(n16, seed=0)
    I.allocate_batch(bf, [16384] * 32, 64)
    with pytest.raises(I.PoolExhausted):
        bf.alloc(256)                               # the 33rd request does not fit


# --- combine ----------------------------------------------------------------------

def test_combine_single_split_is_identity():
    g = np.random.default_rng(1)
    po = g.standard_normal((2, 3, 1, 8)).astype(np.float32)
    pl = g.standard_normal((2, 3, 1)).astype(np.float32)
    o, l = oracle.splitk_combine(po, pl)
    assert np.array_equal(o, po[:, :, 0].astype(np.float64))
    assert np.array_equal(l, pl[:, :, 0].astype(np.float64))


def test_combine_matches_scipy_logsumexp():
    g = np.random.default_rng(2)
    B, H, S, D = 3, 4, 7, 16
    po = g.standard_normal((B, H, S, D)).astype(np.float32)
    pl = (g.standard_normal((B, H, S)) * 30).astype(np.float32)
    pl[0, 0, 2] = -np.inf
    pl[1, 2, :] = -np.inf
    o, l = oracle.splitk_combine(po, pl)
    for b in range(B):
        for h in range(H):
            ls = pl[b, h].astype(np.float64)
            if np.all(ls == -np.inf):
                assert l[b, h] == -np.inf and np.all(o[b, h] == 0)
                continue
            LSE = logsumexp(ls)
            w = np.exp(ls - LSE)
            assert l[b, h] == pytest.approx(LSE, abs=1e-12)
            assert np.allclose(o[b, h], (w[:, None] * po[b, h]).sum(0), rtol=1e-12, atol=1e-12)


def test_combine_status_and_nan():
    po = np.ones((2, 1, 3, 4), np.float32)
    pl = np.zeros((2, 1, 3), np.float32)
    pl[1, 0, 1] = np.nan
    o, l = oracle.splitk_combine(po, pl, status=np.array([4, 0], np.int32))
    assert np.all(o[0] == 0) and l[0, 0] == -np.inf
    assert np.all(np.isnan(o[1])) and np.isnan(l[1, 0])
