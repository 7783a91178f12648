"""Pins for the oracle's paged attention (O5 addressing, O7 attention, O8 combine).

The oracle walks page tables and decodes codes one element at a time; it is
pinned here against a NumPy textbook softmax(qK^T)V computed on pages gathered
by NumPy indexing and decoded by torch's float8_e4m3fn, against closed forms
(single token, uniform scores, all-ones values), physical-page permutation
invariance and split/combine consistency.  The path: the pages' decode-phase
attention over a paged cache stored as e4m3 and converted on read (Cloudflare,
"Smaller, faster, safer: running Kimi and GLM at scale", section "KV 缓存量化"
/ KV cache quantization), with pages mapped per sequence (remio.ai analysis,
shared KV cache safety section).
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from paged_attention_fp8_amd import inputs as I
from helpers import dense_kv, oracle_pool, textbook_attention

SMALL = I.Workload("small_gqa2_ragged", 3, 4, 2, 64, 16, 1, 70, pool_factor=1.5)


def _inputs(w=SMALL, seed=1, **kw):
    return I.make_decode_inputs(w, seed, **kw)


@pytest.mark.parametrize("kv_dtype", [oracle.KV_FP8, oracle.KV_BF16])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_attention_matches_textbook(kv_dtype, seed):
    inp = _inputs(seed=seed)
    pool = oracle_pool(inp, kv_dtype)
    sm = 1.0 / math.sqrt(SMALL.head_dim)
    ks = inp.k_scale if kv_dtype == oracle.KV_FP8 else None
    vs = inp.v_scale if kv_dtype == oracle.KV_FP8 else None
    out, lse = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                      sm, ks, vs)
    for b in range(inp.batch.batch):
        L = int(inp.batch.context_lens[b])
        K, V = dense_kv(pool, inp.batch.page_table[b], L, kv_dtype, ks, vs)
        ro, rl = textbook_attention(inp.q[b], K, V, sm)
        assert np.allclose(out[b], ro, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse[b], rl, rtol=1e-12, atol=1e-12)


def test_gqa_head_mapping_is_floor_division():
    # heads 2g and 2g+1 read KV head g: swapping the two KV heads' data must
    # swap the outputs of the two head pairs
    inp = _inputs(seed=4)
    pool = oracle_pool(inp, oracle.KV_BF16)
    sm = 0.2
    out, _ = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens, sm)
    pool2 = oracle_pool(inp, oracle.KV_BF16)
    pool2.k = np.ascontiguousarray(pool2.k[:, ::-1])
    pool2.v = np.ascontiguousarray(pool2.v[:, ::-1])
    q2 = np.ascontiguousarray(inp.q[:, [2, 3, 0, 1]])
    out2, _ = oracle.paged_attention(pool2, q2, inp.batch.page_table, inp.batch.context_lens, sm)
    assert np.array_equal(out2[:, [2, 3, 0, 1]], out)


def test_softmax_weights_sum_to_one_all_ones_values():
    # V = 1 everywhere (code 0x38 with scale 1): out = sum_t p_t = 1 for every d
    inp = _inputs(seed=5)
    pool = oracle_pool(inp, oracle.KV_FP8)
    pool.v[:] = 0x38
    ones = np.ones(SMALL.kv_heads, np.float32)
    out, _ = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                    0.3, inp.k_scale, ones)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-13)


def test_single_token_returns_its_value():
    inp = _inputs(I.scaled(SMALL, min_len=1, max_len=1), seed=6)
    pool = oracle_pool(inp, oracle.KV_FP8)
    out, lse = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                      0.17, inp.k_scale, inp.v_scale)
    for b in range(inp.batch.batch):
        K, V = dense_kv(pool, inp.batch.page_table[b], 1, oracle.KV_FP8, inp.k_scale, inp.v_scale)
        for h in range(SMALL.q_heads):
            assert np.array_equal(out[b, h], V[0, h // SMALL.group])
            q = I.bf16_bits_to_f32(inp.q[b, h]).astype(np.float64)
            assert lse[b, h] == pytest.approx(0.17 * float(K[0, h // SMALL.group] @ q), abs=1e-12)


def test_zero_query_gives_mean_value_and_log_length():
    inp = _inputs(seed=7)
    pool = oracle_pool(inp, oracle.KV_FP8)
    q = np.zeros_like(inp.q)
    out, lse = oracle.paged_attention(pool, q, inp.batch.page_table, inp.batch.context_lens, 0.5,
                                      inp.k_scale, inp.v_scale)
    for b in range(inp.batch.batch):
        L = int(inp.batch.context_lens[b])
        _, V = dense_kv(pool, inp.batch.page_table[b], L, oracle.KV_FP8, inp.k_scale, inp.v_scale)
        for h in range(SMALL.q_heads):
            assert np.allclose(out[b, h], V[:, h // SMALL.group].mean(0), rtol=1e-12, atol=1e-12)
            assert lse[b, h] == pytest.approx(math.log(L), abs=1e-12)


def test_physical_page_permutation_invariance():
    """Moving pages to other physical slots (and rewriting the tables) must not
    change a single bit of the result."""
    inp = _inputs(seed=8)
    pool = oracle_pool(inp, oracle.KV_FP8)
    sm = 0.25
    args = (inp.k_scale, inp.v_scale)
    out, lse = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                      sm, *args)
    perm = np.random.default_rng(0).permutation(pool.num_pages)      # old page p -> new slot perm[p]
    pool2 = oracle.Pool(oracle.KV_FP8, pool.num_pages, pool.Hkv, pool.P, pool.D)
    pool2.k[perm] = pool.k
    pool2.v[perm] = pool.v
    table2 = np.where(inp.batch.page_table >= 0, perm[np.maximum(inp.batch.page_table, 0)], -1)
    out2, lse2 = oracle.paged_attention(pool2, inp.q, table2, inp.batch.context_lens, sm, *args)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_split_ranges_combine_to_whole():
    """Attention over page-aligned token ranges, merged by the combine, equals
    attention over the whole context."""
    inp = _inputs(I.scaled(SMALL, min_len=50, max_len=70), seed=9)
    pool = oracle_pool(inp, oracle.KV_FP8)
    sm = 0.3
    args = (inp.k_scale, inp.v_scale)
    out, lse = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                      sm, *args)
    B, Hq, D = inp.q.shape
    P = SMALL.page_size
    S = 4
    part_o = np.zeros((B, Hq, S, D), np.float32)
    part_l = np.full((B, Hq, S), -np.inf, np.float32)
    parts64 = {}
    for b in range(B):
        L = int(inp.batch.context_lens[b])
        n = I.pages_needed(L, P)
        cuts = [0, 1, n // 2, n - 1, n]          # includes an empty range when n is small
        for h in range(Hq):
            for s in range(S):
                t0, t1 = cuts[s] * P, min(cuts[s + 1] * P, L)
                o, l = oracle.attention_range(pool, inp.q, inp.batch.page_table, b, h, t0, t1, sm,
                                              *args)
                parts64[b, h, s] = (o, l)
                part_o[b, h, s] = o
                part_l[b, h, s] = l
    # fp64 merge of fp64 partials: exact up to rounding
    for (b, h), _ in np.ndenumerate(np.zeros((B, Hq))):
        ls = np.array([parts64[b, h, s][1] for s in range(S)])
        LSE = logsumexp(ls)
        merged = sum(np.exp(parts64[b, h, s][1] - LSE) * parts64[b, h, s][0]
                     for s in range(S) if np.isfinite(parts64[b, h, s][1]))
        assert LSE == pytest.approx(lse[b, h], abs=1e-12)
        assert np.allclose(merged, out[b, h], rtol=1e-12, atol=1e-12)
    # the oracle's combine on fp32 partials: within fp32 rounding of the whole
    co, cl = oracle.splitk_combine(part_o, part_l)
    assert np.allclose(co, out, rtol=1e-6, atol=1e-6)
    assert np.allclose(cl, lse, rtol=1e-6, atol=1e-6)


def test_aborted_and_invalid_requests():
    inp = _inputs(seed=10)
    pool = oracle_pool(inp, oracle.KV_FP8)
    sm = 0.3
    args = (inp.k_scale, inp.v_scale)
    status = np.array([0, oracle.REQ_TAG_MISMATCH, 0], np.int32)
    out, lse = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                      sm, *args, status=status)
    ref, rl = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                     sm, *args)
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)
    assert np.array_equal(out[[0, 2]], ref[[0, 2]])
    # without a tracker: a bad page id yields NaN, an empty request 0 / -inf
    table = inp.batch.page_table.copy()
    table[0, 0] = inp.num_pages + 3
    lens = inp.batch.context_lens.copy()
    lens[2] = 0
    out2, lse2 = oracle.paged_attention(pool, inp.q, table, lens, sm, *args)
    assert np.all(np.isnan(out2[0])) and np.all(np.isnan(lse2[0]))
    assert np.all(out2[2] == 0) and np.all(lse2[2] == -np.inf)
    assert np.array_equal(out2[1], ref[1])


def test_unused_slots_are_never_read():
    """Poisoned (NaN-coded) slots beyond each context and in free pages do not
    reach the result."""
    inp = _inputs(seed=11)
    clean = oracle_pool(inp, oracle.KV_FP8, poison=False)
    dirty = oracle_pool(inp, oracle.KV_FP8, poison=True)
    a = oracle.paged_attention(clean, inp.q, inp.batch.page_table, inp.batch.context_lens, 0.2,
                               inp.k_scale, inp.v_scale)
    b = oracle.paged_attention(dirty, inp.q, inp.batch.page_table, inp.batch.context_lens, 0.2,
                               inp.k_scale, inp.v_scale)
    assert np.array_equal(a[0], b[0]) and np.all(np.isfinite(b[0]))
