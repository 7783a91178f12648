"""GPU parity of paged decode attention (e4m3 and bf16 pools) through the C
ABI, against the fp64 oracle on the same seeded inputs and identical caches.

Bar (from the path's target): element-wise |gpu - oracle| <= 2e-3 + 1e-2*|oracle|
for out and lse, with fp32 accumulation; caches must be byte-identical first.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_attention_fp8_amd import harness as H
from paged_attention_fp8_amd import inputs as I
from paged_attention_fp8_amd import ops
from helpers import allclose_report, oracle_pool

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATOL, RTOL = 2e-3, 1e-2


def say(*a):
    print(*a, flush=True)


def run_gpu(step, sm, num_splits, check=True, fused=False):
    out, lse, status = H.decode_step(step, sm, num_splits, check=check, fused=fused)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), (None if status is None else status.cpu().numpy())


def pools_equal(step, ref, kv_dtype):
    k, v = step.cache.k_pool.cpu(), step.cache.v_pool.cpu()
    if kv_dtype == ops.KV_BF16:
        k = k.view(torch.int16).numpy().view(np.uint16)
        v = v.view(torch.int16).numpy().view(np.uint16)
    else:
        k, v = k.numpy(), v.numpy()
    return np.array_equal(k, ref.k) and np.array_equal(v, ref.v)


def compare(out, lse, ro, rl, what):
    ok1, ma, mr = allclose_report(out, ro, ATOL, RTOL)
    ok2, la, lr = allclose_report(lse, rl, ATOL, RTOL)
    say(f"  {what}: out max_abs={ma:.3e} max_rel={mr:.3e}; lse max_abs={la:.3e}")
    assert ok1 and ok2, f"{what}: out max_abs={ma} rel={mr}, lse max_abs={la} rel={lr}"


CASES = [
    # name, B, Hq, Hkv, D, P, min_len, max_len
    I.Workload("mha_d64_p16_ragged", 3, 4, 4, 64, 16, 1, 300, pool_factor=1.5),
    I.Workload("mha_d128_p64", 2, 2, 2, 128, 64, 100, 700, pool_factor=1.5),
    I.Workload("gqa2_d128_p16", 2, 4, 2, 128, 16, 200, 450, pool_factor=1.5),
    I.Workload("gqa4_d128_p16_outliers", 3, 16, 4, 128, 16, 250, 1100, pool_factor=1.3,
               outlier_frac=0.01, outlier_mult=20.0),
    I.Workload("gqa8_d128_p64_ragged", 4, 16, 2, 128, 64, 1, 1500, pool_factor=1.3),
    I.Workload("gqa16_d64_p32", 2, 32, 2, 64, 32, 300, 900, pool_factor=1.3),
    I.Workload("gqa5_d128_p256", 2, 10, 2, 128, 256, 700, 1300, pool_factor=1.3),
    I.Workload("gqa8_d64_p128_short", 5, 8, 1, 64, 128, 1, 70, pool_factor=2.0),
    I.Workload("gqa16_d128_p64", 2, 32, 2, 128, 64, 200, 800, pool_factor=1.3),   # the largest group
]


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("splits", [1, 3])
def test_attention_matches_oracle(w, kv_dtype, splits):
    say(f"attn: {w.name} dtype={kv_dtype} splits={splits}")
    inp = I.make_decode_inputs(w, 11)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    out, lse, status = run_gpu(step, sm, splits)
    assert np.all(status == 0)
    ref = oracle_pool(inp, kv_dtype, poison=True)
    assert pools_equal(step, ref, kv_dtype), "caches differ"
    ks = inp.k_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    vs = inp.v_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    ro, rl = oracle.paged_attention(ref, inp.q, inp.batch.page_table, inp.batch.context_lens, sm,
                                    ks, vs)
    compare(out, lse, ro, rl, w.name)


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("groups", [1, 3, 40])
def test_balanced_matches_oracle(w, kv_dtype, groups):
    """The balanced partition (num_splits = -W): one work-group per head
    (every request written whole), ranges that cut requests, and more
    work-groups than pages (empty ranges)."""
    say(f"attn balanced: {w.name} dtype={kv_dtype} W={groups}")
    inp = I.make_decode_inputs(w, 21)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    out, lse, status = run_gpu(step, sm, -groups)
    assert np.all(status == 0)
    ref = oracle_pool(inp, kv_dtype, poison=True)
    assert pools_equal(step, ref, kv_dtype), "caches differ"
    ks = inp.k_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    vs = inp.v_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    ro, rl = oracle.paged_attention(ref, inp.q, inp.batch.page_table, inp.batch.context_lens, sm,
                                    ks, vs)
    compare(out, lse, ro, rl, f"{w.name} W={groups}")


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
def test_large_batch_matches_oracle(kv_dtype):
    """999 short ragged requests (1-300 tokens, GQA 16/2, 16-token pages):
    launch grids of 1998 to 5994 work-groups, not multiples of the 8 XCDs
    they are dealt to, at the library's default split, 3 splits, and the
    balanced partition (whose work-groups scan all 999 lengths)."""
    w = I.Workload("many_short", 999, 16, 2, 128, 16, 1, 300, pool_factor=1.3)
    say(f"attn large batch: dtype={kv_dtype}")
    inp = I.make_decode_inputs(w, 31)
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    ref = None
    for splits in (0, 3, -ops.default_balanced_groups(w.kv_heads)):
        out, lse, status = run_gpu(step, sm, splits)
        assert np.all(status == 0)
        if ref is None:
            ref = oracle_pool(inp, kv_dtype, poison=True)
            assert pools_equal(step, ref, kv_dtype), "caches differ"
            ks = inp.k_scale if kv_dtype == ops.KV_FP8_E4M3 else None
            vs = inp.v_scale if kv_dtype == ops.KV_FP8_E4M3 else None
            ro, rl = oracle.paged_attention(ref, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                            sm, ks, vs)
        compare(out, lse, ro, rl, f"999 requests, splits={splits}")


def test_balanced_edge_requests():
    """Balanced partition with aborted, empty and invalid requests between live
    ones, a page id outside the pool inside a cut request, and the library's
    default W: aborted and empty rows give 0 / -inf, invalid ones NaN, the bad
    page's request NaN, and every other row matches the oracle."""
    w = CASES[4]
    inp = I.make_decode_inputs(w, 22)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    ops.kv_quant_append(step.cache, step.batch, step.k_new, step.v_new)
    order = [0, 1, 2, 3, 0, 1, 2, 3]
    q = step.q[order].contiguous()
    pt = step.batch.page_table[order].clone()
    lens = step.batch.context_lens[order].clone()
    status = torch.zeros(8, dtype=torch.int32, device=DEV)
    status[1] = 3                                   # aborted
    lens[2] = 0                                     # empty
    lens[5] = pt.shape[1] * w.page_size + 1         # past the table: invalid
    live = [0, 3, 4, 6, 7]
    bad_row = max(live, key=lambda r: int(lens[r]))
    assert int(lens[bad_row]) > w.page_size
    pt[bad_row, 1] = step.cache.num_pages + 7       # outside the pool, in page 1 of the longest
    batch = ops.DecodeBatch(pt, lens, status)
    want = oracle.paged_attention(oracle_pool(inp, oracle.KV_FP8), inp.q[order], pt.cpu().numpy(),
                                  lens.cpu().numpy(), 0.09, inp.k_scale, inp.v_scale,
                                  status=status.cpu().numpy())
    for groups in (2, 5, ops.default_balanced_groups(w.kv_heads)):
        out, lse = ops.paged_decode_attn(step.cache, batch, q, 0.09, -groups)
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        say(f"  balanced edges W={groups}")
        for b in (1, 2):
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b])), b
        assert np.all(np.isnan(out[5])) and np.all(np.isnan(lse[5]))
        assert np.all(np.isnan(out[bad_row])) and np.all(np.isnan(lse[bad_row]))
        good = [b for b in range(8) if b not in (1, 2, 5, bad_row)]
        compare(out[good], lse[good], want[0][good], want[1][good], f"edges W={groups}")


def test_balanced_against_uniform_splits_and_deterministic():
    """Same attention as the uniform split path up to the rounding of P
    against different running maxima (bound as in the split-invariance test),
    and bitwise repeatable."""
    w = CASES[4]
    inp = I.make_decode_inputs(w, 23)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    ops.kv_quant_append(step.cache, step.batch, step.k_new, step.v_new)
    base = [t.cpu().numpy() for t in ops.paged_decode_attn(step.cache, step.batch, step.q, 0.09, 1)]
    vmax = 448.0 * float(inp.v_scale.max())
    bound = 2.0 ** -14 * vmax + 1e-6
    for groups in (2, 7, 64):
        a = [t.cpu().numpy() for t in ops.paged_decode_attn(step.cache, step.batch, step.q, 0.09, -groups)]
        b = [t.cpu().numpy() for t in ops.paged_decode_attn(step.cache, step.batch, step.q, 0.09, -groups)]
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), groups
        diff = np.abs(a[0] - base[0]).max()
        say(f"  balanced W={groups} vs S=1: max |diff| = {diff:.3e} (bound {bound:.3e})")
        assert diff <= bound
        assert np.allclose(a[1], base[1], rtol=1e-5, atol=1e-5)


def test_default_split_choice_matches_oracle():
    w = CASES[4]
    inp = I.make_decode_inputs(w, 12)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    sm = 0.088
    out, lse, _ = run_gpu(step, sm, 0)
    ref = oracle_pool(inp, oracle.KV_FP8)
    ro, rl = oracle.paged_attention(ref, inp.q, inp.batch.page_table, inp.batch.context_lens, sm,
                                    inp.k_scale, inp.v_scale)
    compare(out, lse, ro, rl, "default splits")


def test_softmax_weights_sum_to_one():
    """With every V = 1 (code 0x38, scale 1) the output is sum_t p_t = 1."""
    w = CASES[3]
    inp = I.make_decode_inputs(w, 13)
    inp.v_scale[:] = 1.0
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    ops.kv_quant_append(step.cache, step.batch, step.k_new, step.v_new)
    step.cache.v_pool.fill_(0x38)
    out, lse = ops.paged_decode_attn(step.cache, step.batch, step.q, 0.1, 2)
    o = out.cpu().numpy()
    assert np.abs(o - 1.0).max() < 1e-4, np.abs(o - 1.0).max()


def test_determinism_and_split_invariance():
    w = CASES[4]
    inp = I.make_decode_inputs(w, 14)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    ops.kv_quant_append(step.cache, step.batch, step.k_new, step.v_new)
    runs = {}
    for S in (1, 2, 5, 24):
        a = ops.paged_decode_attn(step.cache, step.batch, step.q, 0.09, S)
        b = ops.paged_decode_attn(step.cache, step.batch, step.q, 0.09, S)
        a = [t.cpu().numpy() for t in a]
        b = [t.cpu().numpy() for t in b]
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), f"S={S} not deterministic"
        runs[S] = a
    # different splits split P into bf16 high + low parts against different
    # running maxima: each run's P carries a relative error <= 2^-16, so two
    # runs differ by at most 2^-15 * max|v|, plus fp32 summation in another
    # order (a few 2^-24 per step); 2^-14 * max|v| covers both, far inside
    # the parity tolerance
    vmax = 448.0 * float(inp.v_scale.max())
    bound = 2.0 ** -14 * vmax + 1e-6
    for S in (2, 5, 24):
        diff = np.abs(runs[S][0] - runs[1][0]).max()
        say(f"  split {S} vs 1: max |diff| = {diff:.3e} (bound {bound:.3e})")
        assert diff <= bound
        assert np.allclose(runs[S][1], runs[1][1], rtol=1e-5, atol=1e-5)


def test_physical_page_permutation_is_bitwise_invariant():
    w = CASES[3]
    inp = I.make_decode_inputs(w, 15)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    ops.kv_quant_append(step.cache, step.batch, step.k_new, step.v_new)
    a = [t.cpu().numpy() for t in ops.paged_decode_attn(step.cache, step.batch, step.q, 0.09, 3)]
    n = step.cache.num_pages
    perm = torch.from_numpy(np.random.default_rng(1).permutation(n)).to(DEV)
    k2 = torch.empty_like(step.cache.k_pool)
    v2 = torch.empty_like(step.cache.v_pool)
    k2[perm] = step.cache.k_pool
    v2[perm] = step.cache.v_pool
    pt = step.batch.page_table
    pt2 = torch.where(pt >= 0, perm[pt.clamp(min=0).long()].to(torch.int32), pt).contiguous()
    cache2 = ops.PagedKVCache(k2, v2, step.cache.k_scale, step.cache.v_scale)
    b2 = ops.DecodeBatch(pt2, step.batch.context_lens)
    c = [t.cpu().numpy() for t in ops.paged_decode_attn(cache2, b2, step.q, 0.09, 3)]
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


@pytest.mark.parametrize("fused", [False, True], ids=["check_then_append", "append_checked"])
@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
def test_stale_request_aborted_and_excluded(kv_dtype, fused):
    """A request with a stale tag is flagged, not appended, outputs 0 / -inf,
    and the other requests are bitwise what they are without it; its pages
    may hold anything (NaN codes here) without effect.  Same with the check
    fused into the append launch."""
    w = I.scaled(CASES[4], stale_requests=1)
    inp = I.make_decode_inputs(w, 16)
    assert len(inp.stale) == 1
    bad = inp.stale[0]
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    # poison the stale request's pages
    rows = inp.batch.page_table[bad]
    rows = rows[rows >= 0]
    nan = H.FP8_NAN_CODE if kv_dtype == ops.KV_FP8_E4M3 else H.BF16_NAN_BITS
    idx = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    if kv_dtype == ops.KV_FP8_E4M3:
        step.cache.k_pool[idx] = nan
        step.cache.v_pool[idx] = nan
    else:
        step.cache.k_pool.view(torch.int16)[idx] = nan
        step.cache.v_pool.view(torch.int16)[idx] = nan
    out, lse, status = run_gpu(step, 0.088, 3, fused=fused)
    want = np.zeros(inp.batch.batch, np.int32)
    want[bad] = oracle.REQ_TAG_MISMATCH
    assert np.array_equal(status, want)
    assert np.all(out[bad] == 0) and np.all(np.isneginf(lse[bad]))
    others = [b for b in range(inp.batch.batch) if b != bad]
    # the same step without the aborted request
    sub = ops.DecodeBatch(step.batch.page_table[others].contiguous(),
                          step.batch.context_lens[others].contiguous())
    o2, l2 = ops.paged_decode_attn(step.cache, sub, step.q[others].contiguous(), 0.088, 3)
    assert np.array_equal(out[others], o2.cpu().numpy())
    assert np.array_equal(lse[others], l2.cpu().numpy())
    ref = oracle_pool(inp, kv_dtype, poison=True)
    ks = inp.k_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    vs = inp.v_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    ro, rl = oracle.paged_attention(ref, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                    0.088, ks, vs, status=want)
    compare(out[others], lse[others], ro[others], rl[others], "stale excluded")


def test_no_tracker_invalid_inputs_do_not_fault():
    """Without a status array: a page id outside the pool or a length past the
    table gives NaN rows; length 0 gives 0 / -inf; other rows are unaffected."""
    w = CASES[1]
    inp = I.make_decode_inputs(w, 17)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    ops.kv_quant_append(step.cache, step.batch, step.k_new, step.v_new)
    B = 4
    q = step.q[[0, 1, 0, 1]].contiguous()
    pt = step.batch.page_table[[0, 1, 0, 1]].clone()
    lens = step.batch.context_lens[[0, 1, 0, 1]].clone()
    pt[0, 0] = step.cache.num_pages + 5
    lens[2] = 0
    lens[3] = pt.shape[1] * w.page_size + 1
    out, lse = ops.paged_decode_attn(step.cache, ops.DecodeBatch(pt, lens), q, 0.09, 2)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isnan(out[3]))
    ref, _ = ops.paged_decode_attn(step.cache, step.batch, step.q, 0.09, 2)
    assert np.array_equal(out[1], ref.cpu().numpy()[1])
    ro, rl = oracle.paged_attention(oracle_pool(inp, oracle.KV_FP8), inp.q[[0, 1, 0, 1]],
                                    pt.cpu().numpy(), lens.cpu().numpy(), 0.09, inp.k_scale,
                                    inp.v_scale)
    assert np.array_equal(np.isnan(ro), np.isnan(out))


def test_empty_batch_is_a_no_op():
    w = CASES[0]
    inp = I.make_decode_inputs(w, 18)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    empty = ops.DecodeBatch(step.batch.page_table[:0].contiguous(),
                            step.batch.context_lens[:0].contiguous())
    out, lse = ops.paged_decode_attn(step.cache, empty, step.q[:0].contiguous(), 0.1, 1)
    assert out.shape == (0, w.q_heads, w.head_dim)


def test_host_errors_are_reported():
    w = CASES[2]
    inp = I.make_decode_inputs(w, 19)
    step = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    with pytest.raises(ops.Pafp8Error, match="sm_scale"):
        ops.paged_decode_attn(step.cache, step.batch, step.q, -1.0, 1)
    q33 = torch.zeros((2, 34, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops.Pafp8Error, match="group size"):
        ops.paged_decode_attn(step.cache, step.batch, q33[:, :34].contiguous(), 0.1, 1)
    with pytest.raises(ops.Pafp8Error, match="at most 65536"):
        ops.paged_decode_attn(step.cache, step.batch, step.q, 0.1, -65537)
    need = ops.workspace_bytes(step.batch.batch, w.q_heads, w.head_dim, -8)
    with pytest.raises(ops.Pafp8Error, match="workspace"):
        ops.paged_decode_attn(step.cache, step.batch, step.q, 0.1, -8,
                              torch.empty(need - 16, dtype=torch.uint8, device=DEV))
