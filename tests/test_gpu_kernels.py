"""GPU parity of the exact (integer / byte) parts of the path, through the C ABI:
the e4m3 codec, the page-tag check, quantise-on-write, and the split-K combine.

Bar: bit-exact against the oracle for codes, pools and request status; the
combine (float) within max-abs 2e-3 / rel 1e-2 (in practice ~1e-6).
"""

import numpy as np
import pytest
import torch

import oracle
from paged_attention_fp8_amd import harness as H
from paged_attention_fp8_amd import inputs as I
from paged_attention_fp8_amd import ops
from helpers import allclose_report, oracle_pool, poison_value

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


# --- codec ------------------------------------------------------------------------

def test_decode_all_codes_every_route():
    say("codec: decode 256 codes")
    codes = torch.arange(256, dtype=torch.uint8, device=DEV)
    f32, via16, viabf = (t.cpu().numpy().astype(np.float64) for t in ops.e4m3_decode(codes))
    ref = oracle.e4m3_decode_table()
    for got in (f32, via16, viabf):
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.array_equal(got[fin], ref[fin])
        assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_encode_golden_and_specials():
    say("codec: encode anchors")
    import os
    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "e4m3_encode_anchors.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                v, c = line.split()[:2]
                rows.append((np.float32(float(v)), int(c, 16)))
    x = torch.tensor([r[0] for r in rows], dtype=torch.float32, device=DEV)
    got = ops.e4m3_encode(x).cpu().numpy()
    assert got.tolist() == [r[1] for r in rows]


def test_encode_all_fp32_bit_patterns():
    """Every one of the 2^32 fp32 inputs encodes exactly as the oracle does."""
    chunk = 1 << 28
    for k in range(1 << 32 >> 28):
        first = k * chunk
        say(f"codec: encode sweep chunk {k} first=0x{first:08x}")
        start = first - (1 << 31)      # int32 view of the same bit patterns
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device=DEV).to(torch.int32)
        codes = ops.e4m3_encode(bits.view(torch.float32)).cpu().numpy()
        del bits
        ref = oracle.e4m3_encode_bits_range((first ^ 0x80000000) & 0xFFFFFFFF, chunk)
        if not np.array_equal(codes, ref):
            bad = np.flatnonzero(codes != ref)[:5]
            pats = [hex(((first ^ 0x80000000) + int(i)) & 0xFFFFFFFF) for i in bad]
            raise AssertionError(f"encode mismatch at fp32 patterns {pats}: "
                                 f"gpu {codes[bad].tolist()} oracle {ref[bad].tolist()}")


# --- page-tag check -----------------------------------------------------------------

def _check_case(pool, batch, lens, P):
    dbatch, tags, exp = H.upload_batch(I.PagedBatch(P, batch.page_table, lens, batch.expected_tags),
                                       pool, DEV)
    got = ops.page_tag_check(dbatch, P, tags, exp).cpu().numpy()
    want = oracle.page_tag_check(batch.page_table, lens, batch.expected_tags, pool.tags, P)
    assert np.array_equal(got, want), (got, want)
    return got


def test_tag_check_injected_failures():
    say("tag check: injected stale / oob / bad length")
    P = 16
    pool = I.PagePool(1000, seed=2)
    lens = np.array([40, 200, 16, 1, 500, 77, 300, 64], np.int32)
    batch = I.allocate_batch(pool, lens, P)
    I.make_stale(pool, batch, 1, 5)
    I.make_stale(pool, batch, 6, 0)
    batch.page_table[3, 0] = 1000
    batch.page_table[4, 2] = -7
    I.make_stale(pool, batch, 4, 3)
    lens2 = lens.copy()
    lens2[5] = 0
    lens2[7] = batch.max_pages * P + 1
    got = _check_case(pool, batch, lens2, P)
    assert got.tolist() == [0, 1, 0, 2, 3, 4, 1, 4]


@pytest.mark.parametrize("P", [16, 64, 256])
def test_tag_check_random(P):
    g = np.random.default_rng(P)
    for trial in range(6):
        B = int(g.integers(1, 300))
        pool = I.PagePool(int(g.integers(4000, 20000)), seed=trial)
        lens = g.integers(0, 40 * P, B).astype(np.int32)
        lens = np.maximum(lens, 1)
        try:
            batch = I.allocate_batch(pool, lens, P)
        except I.PoolExhausted:
            continue
        for _ in range(int(g.integers(0, 8))):
            b = int(g.integers(0, B))
            I.make_stale(pool, batch, b, int(g.integers(0, I.pages_needed(lens[b], P))))
        lens[g.random(B) < 0.05] = 0
        say(f"tag check: random P={P} trial={trial} B={B}")
        _check_case(pool, batch, lens, P)


def test_tag_check_thousand_requests_one_stale():
    say("tag check: 1000 x 4096 pages, one stale")
    P = 64
    pool = I.PagePool(1000 * 4096, seed=5, order="sequential")
    batch = I.allocate_batch(pool, np.full(1000, 4096 * 64, np.int32), P)
    I.make_stale(pool, batch, 613, 4000)
    got = _check_case(pool, batch, batch.context_lens, P)
    assert np.flatnonzero(got).tolist() == [613]


# --- quantise-on-write ----------------------------------------------------------------

WRITE_CASES = [
    I.Workload("w_d64_p16", 3, 4, 4, 64, 16, 1, 100, pool_factor=1.5),
    I.Workload("w_d128_p64", 4, 16, 8, 128, 64, 60, 300, pool_factor=1.3),
    I.Workload("w_d128_p32_outliers", 2, 8, 2, 128, 32, 200, 333, pool_factor=1.2,
               outlier_frac=0.01, outlier_mult=20.0),
    I.Workload("w_d64_p256", 2, 2, 1, 64, 256, 17, 600, pool_factor=2.0),
]


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16])
@pytest.mark.parametrize("w", WRITE_CASES, ids=lambda w: w.name)
def test_fill_and_append_pools_bit_exact(w, kv_dtype):
    say(f"kv write: {w.name} dtype={kv_dtype}")
    inp = I.make_decode_inputs(w, 7)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    ops.kv_quant_append(step.cache, step.batch, step.k_new, step.v_new)
    ref = oracle_pool(inp, kv_dtype, poison=True)
    k = step.cache.k_pool.cpu()
    v = step.cache.v_pool.cpu()
    if kv_dtype == ops.KV_BF16:
        k, v = k.view(torch.int16).numpy().view(np.uint16), v.view(torch.int16).numpy().view(np.uint16)
    else:
        k, v = k.numpy(), v.numpy()
    assert np.array_equal(k, ref.k)
    assert np.array_equal(v, ref.v)


@pytest.mark.parametrize("kv_dtype,P,D", [(ops.KV_FP8_E4M3, 16, 64), (ops.KV_FP8_E4M3, 64, 128),
                                          (ops.KV_FP8_E4M3, 128, 128), (ops.KV_BF16, 16, 64),
                                          (ops.KV_BF16, 32, 128), (ops.KV_BF16, 256, 128)])
def test_fill_arbitrary_offsets_and_status(kv_dtype, P, D):
    """Blocks starting at unaligned positions, partial and whole segments,
    clipped counts, aborted and invalid requests."""
    say(f"kv write: offsets / status dtype={kv_dtype} P={P} D={D}")
    L = 300
    w = I.Workload("w", 5, 4, 2, D, P, L, L, pool_factor=1.0)
    inp = I.make_decode_inputs(w, 3)
    fp8 = kv_dtype == ops.KV_FP8_E4M3
    cache = H.new_cache(w, inp.num_pages, kv_dtype, DEV, inp.k_scale if fp8 else None,
                        inp.v_scale if fp8 else None)
    dbatch, _, _ = H.upload_batch(inp.batch, inp.pool, DEV)
    cap = inp.batch.max_pages * P
    status = np.array([0, 1, 0, 0, 0], np.int32)
    start = np.array([3, 0, cap - 10, -5, 33], np.int32)   # cap - 10 runs past the table
    count = np.array([150, 10, 40, 90, 0], np.int32)       # -5 starts before it; 150 is clipped
    T = 130
    k_src = np.stack([inp.k_tokens[b][:T] for b in range(5)])
    v_src = np.stack([inp.v_tokens[b][:T] for b in range(5)])
    db = dbatch.with_status(torch.from_numpy(status).to(DEV))
    ops.kv_quant_fill(cache, db, torch.from_numpy(start).to(DEV), torch.from_numpy(count).to(DEV),
                      H.bf16_tensor(k_src, DEV), H.bf16_tensor(v_src, DEV))
    okv = oracle.KV_FP8 if fp8 else oracle.KV_BF16
    ref = oracle.Pool(okv, inp.num_pages, 2, P, D, fill=poison_value(okv))
    oracle.kv_write(ref, inp.batch.page_table, start, np.minimum(count, T), k_src, v_src,
                    inp.k_scale if fp8 else None, inp.v_scale if fp8 else None, status=status)
    k, v = cache.k_pool.cpu(), cache.v_pool.cpu()
    if not fp8:
        k, v = k.view(torch.int16), v.view(torch.int16)
    k, v = k.numpy(), v.numpy()
    if not fp8:
        k, v = k.view(np.uint16), v.view(np.uint16)
    assert np.array_equal(k, ref.k)
    assert np.array_equal(v, ref.v)


def test_append_skips_aborted_and_invalid_lengths():
    say("kv write: append status / lengths")
    w = I.Workload("w", 4, 4, 2, 128, 16, 30, 30, pool_factor=1.0)
    inp = I.make_decode_inputs(w, 4)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    ref = oracle_pool(inp, oracle.KV_FP8, append=False)
    lens = inp.batch.context_lens.copy()
    lens[2] = 0
    lens[3] = 10_000
    status = np.array([0, 2, 0, 0], np.int32)
    b = ops.DecodeBatch(step.batch.page_table, torch.from_numpy(lens).to(DEV),
                        torch.from_numpy(status).to(DEV))
    ops.kv_quant_append(step.cache, b, step.k_new, step.v_new)
    oracle.kv_append(ref, inp.batch.page_table, lens, inp.k_new(), inp.v_new(), inp.k_scale,
                     inp.v_scale, status=status)
    assert np.array_equal(step.cache.k_pool.cpu().numpy(), ref.k)
    assert np.array_equal(step.cache.v_pool.cpu().numpy(), ref.v)


SCALE_ROUNDS = [
    # fast-path scales, its boundaries, and scales outside it (rescaled form)
    [1.0, 3.7e-3, 0.0137, 2.0 ** -64, 2.0 ** 64, 2.0 ** -70, 5e30, 1.5e-20],
    [0.5, 1.0 / 448, 7.77, 2.0 ** -63.5, 2.0 ** 63.9, 1e-30, 2.0 ** 70, 0.1],
    # negative scales, subnormal scales, the largest finite ones
    [-1.0, -3.7e-3, 1e-40, -2.0 ** 100, 3.0e38, -1e-38, 2.0 ** -126, 2.0 ** -149],
]


@pytest.mark.parametrize("rnd", range(len(SCALE_ROUNDS)))
def test_fill_quantises_every_bf16_pattern(rnd):
    """All 65536 bf16 bit patterns (NaN, infinities, subnormals, zeros
    included) under 16 scales each, through kv_quant_fill: pools byte-exact
    against the oracle, which divides."""
    say(f"kv write: every bf16 pattern, scale round {rnd}")
    Hkv, D, P, T = 8, 128, 64, 512
    w = I.Workload("allbf16", 1, Hkv, Hkv, D, P, T + 1, T + 1, pool_factor=1.0)
    inp = I.make_decode_inputs(w, 5)
    pats = np.arange(65536, dtype=np.uint16).reshape(T, D)
    g = np.random.default_rng(rnd)
    k = np.stack([pats[:, g.permutation(D)] for _ in range(Hkv)], axis=1)[None]   # [1][T][Hkv][D]
    v = np.stack([pats[g.permutation(T)] for _ in range(Hkv)], axis=1)[None]
    ks = np.asarray(SCALE_ROUNDS[rnd], np.float32)
    vs = ks[::-1].copy()
    cache = H.new_cache(w, inp.num_pages, ops.KV_FP8_E4M3, DEV, ks, vs)
    dbatch, _, _ = H.upload_batch(inp.batch, inp.pool, DEV)
    zero = np.zeros(1, np.int32)
    count = np.array([T], np.int32)
    ops.kv_quant_fill(cache, dbatch, torch.from_numpy(zero).to(DEV), torch.from_numpy(count).to(DEV),
                      H.bf16_tensor(k, DEV), H.bf16_tensor(v, DEV))
    ref = oracle.Pool(oracle.KV_FP8, inp.num_pages, Hkv, P, D, fill=H.FP8_NAN_CODE)
    oracle.kv_write(ref, inp.batch.page_table, zero, count, k, v, ks, vs)
    assert np.array_equal(cache.k_pool.cpu().numpy(), ref.k)
    assert np.array_equal(cache.v_pool.cpu().numpy(), ref.v)


# --- fused check + append, device-side reallocation ------------------------------------

def _dev(a, dtype=np.int32):
    return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).to(DEV)


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16])
@pytest.mark.parametrize("D,P", [(64, 16), (128, 64)])
def test_append_checked_equals_check_then_append(kv_dtype, D, P):
    say(f"append checked: dtype={kv_dtype} D={D} P={P}")
    w = I.Workload("chk", 8, 16, 4, D, P, 1, 40 * P, pool_factor=1.5)
    inp = I.make_decode_inputs(w, 11)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    table = inp.batch.page_table.copy()
    lens = inp.batch.context_lens.copy()
    tags = inp.pool.tags.copy()
    tags[table[1, 0]] += np.uint32(1)      # request 1: page 0 reallocated behind its back
    table[3, 0] = inp.num_pages + 5        # request 3: a page id outside the pool
    lens[5] = 0                            # request 5: invalid length
    dbatch = ops.DecodeBatch(_dev(table), _dev(lens))
    got = ops.kv_quant_append_checked(step.cache, dbatch, _dev(tags), step.expected_tags,
                                      step.k_new, step.v_new).cpu().numpy()
    want = oracle.page_tag_check(table, lens, inp.batch.expected_tags, tags, P)
    assert np.array_equal(got, want), (got, want)
    assert want[1] == 1 and want[3] == 2 and want[5] == 4 and np.count_nonzero(want) == 3
    fp8 = kv_dtype == ops.KV_FP8_E4M3
    okv = oracle.KV_FP8 if fp8 else oracle.KV_BF16
    ref = oracle_pool(inp, okv, poison=True, append=False)
    oracle.kv_append(ref, table, lens, inp.k_new(), inp.v_new(), inp.k_scale if fp8 else None,
                     inp.v_scale if fp8 else None, status=want)
    k, v = step.cache.k_pool.cpu(), step.cache.v_pool.cpu()
    if not fp8:
        k, v = k.view(torch.int16), v.view(torch.int16)
    k, v = k.numpy(), v.numpy()
    if not fp8:
        k, v = k.view(np.uint16), v.view(np.uint16)
    assert np.array_equal(k, ref.k)
    assert np.array_equal(v, ref.v)


def test_tag_realloc_matches_oracle():
    say("tag realloc: distinct pages vs oracle")
    g = np.random.default_rng(21)
    num_pages, B, maxP = 5000, 20, 64
    tags0 = g.integers(0, 2**32, num_pages, dtype=np.uint64).astype(np.uint32)
    tags0[:50] = 0xFFFFFFFF
    table0 = g.integers(-1, num_pages, (B, maxP)).astype(np.int32)
    exp0 = g.integers(0, 2**32, (B, maxP), dtype=np.uint64).astype(np.uint32)
    n = 3000
    ids = g.permutation(num_pages)[:n].astype(np.int32)
    ids[::97] = -3                                   # outside the pool
    ids[5::101] = num_pages + 1
    req = np.full(n, -1, np.int32)
    slot = np.full(n, 0, np.int32)
    k = min(n, B * maxP)
    perm = g.permutation(B * maxP)[:k]               # distinct owner slots
    req[:k], slot[:k] = perm // maxP, perm % maxP
    req[g.random(n) < 0.1] = B + 3                   # owners outside the table
    t_d, pt_d, ex_d = _dev(tags0), _dev(table0), _dev(exp0)
    ops.page_tag_realloc(_dev(ids), t_d, _dev(req), _dev(slot), pt_d, ex_d)
    rt, rp, re_ = oracle.page_tag_realloc(ids, tags0, req, slot, table0, exp0)
    assert np.array_equal(t_d.cpu().numpy().view(np.uint32), rt)
    assert np.array_equal(pt_d.cpu().numpy(), rp)
    assert np.array_equal(ex_d.cpu().numpy().view(np.uint32), re_)


def test_tag_realloc_repeated_pages():
    """A page listed m times moves on by m; its owners record m distinct
    tags, one per listing."""
    say("tag realloc: repeated pages")
    tags0 = np.array([10, 0xFFFFFFFE, 3], np.uint32)
    ids = np.array([1, 1, 1, 0, 1], np.int32)
    B, maxP = 1, 5
    req = np.zeros(5, np.int32)
    slot = np.arange(5, dtype=np.int32)
    t_d, ex_d = _dev(tags0), _dev(np.zeros((B, maxP), np.uint32))
    ops.page_tag_realloc(_dev(ids), t_d, _dev(req), _dev(slot), None, ex_d)
    tags = t_d.cpu().numpy().view(np.uint32)
    ex = ex_d.cpu().numpy().view(np.uint32)[0]
    assert list(tags) == [11, 2, 3]
    assert sorted(ex[[0, 1, 2, 4]].tolist()) == [0, 1, 2, 0xFFFFFFFF] and ex[3] == 11


# --- combine --------------------------------------------------------------------------

@pytest.mark.parametrize("S,D", [(1, 128), (7, 64), (16, 128), (17, 64), (33, 64), (64, 128), (130, 128),
                                 (256, 128), (257, 64), (5, 96), (70, 256)])
def test_combine_matches_oracle(S, D):
    say(f"combine: S={S} D={D}")
    g = np.random.default_rng(S * 1000 + D)
    B, Hq = 3, 5
    po = g.standard_normal((B, Hq, S, D)).astype(np.float32)
    pl = (g.standard_normal((B, Hq, S)) * 8).astype(np.float32)
    pl[g.random((B, Hq, S)) < 0.2] = -np.inf
    pl[0, 1, :] = -np.inf
    po[pl == -np.inf] = 0.0
    if S > 1:
        pl[2, 3, 1] = np.nan
    status = np.array([0, 4, 0], np.int32)
    out, lse = ops.splitk_combine(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV),
                                  torch.from_numpy(status).to(DEV))
    ro, rl = oracle.splitk_combine(po, pl, status)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(np.isnan(out), np.isnan(ro)) and np.array_equal(np.isnan(lse), np.isnan(rl))
    fin = ~np.isnan(ro)
    ok, ma, mr = allclose_report(out[fin], ro[fin])
    assert ok, (ma, mr)
    finl = np.isfinite(rl)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    assert np.allclose(lse[finl], rl[finl], rtol=1e-5, atol=1e-5)
