"""Host-side input recipe: bf16 rounding, determinism, the page pool."""
import numpy as np
import pytest
import torch

from paged_attention_fp8_amd import inputs as I


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100_000).astype(np.float32) * 100,
                        g.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40], np.float32)])
    fin = np.isfinite(x)
    ours = I.f32_to_bf16_bits(x[fin])
    ref = torch.from_numpy(x[fin]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = I.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(I.bf16_bits_to_f32(nan))[0]


def test_inputs_are_deterministic_per_seed():
    w = I.scaled(I.WORKLOADS["gqa4_4k_outliers"], batch=2, min_len=100, max_len=100)
    a = I.make_decode_inputs(w, 42)
    b = I.make_decode_inputs(w, 42)
    c = I.make_decode_inputs(w, 43)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_tokens[1], b.k_tokens[1])
    assert np.array_equal(a.batch.page_table, b.batch.page_table)
    assert not np.array_equal(a.q, c.q)


def test_outlier_scale_uses_bulk_amax():
    w = I.scaled(I.WORKLOADS["gqa4_4k_outliers"], batch=2, min_len=512, max_len=512)
    inp = I.make_decode_inputs(w, 1)
    allk = np.concatenate([I.bf16_bits_to_f32(k) for k in inp.k_tokens])
    amax_all = np.abs(allk).max(axis=(0, 2))
    assert np.all(amax_all > 448 * inp.k_scale)    # outliers exceed the range: saturation
    assert np.all(inp.k_scale > 0) and inp.k_scale.dtype == np.float32


def test_scale_closed_form():
    s = I.fp8_scale_from_amax([448.0, 4.48, 0.0])
    assert s[0] == np.float32(1.0) and s[1] == np.float32(4.48) / np.float32(448) and s[2] == 1.0


def test_page_pool_alloc_tags_and_exhaustion():
    pool = I.PagePool(10, seed=3)
    a, ta = pool.alloc(4)
    b, tb = pool.alloc(6)
    assert len(set(a.tolist()) | set(b.tolist())) == 10
    assert np.all(ta == 1) and np.all(tb == 1)
    with pytest.raises(I.PoolExhausted):
        pool.alloc(1)
    pool.release(a[:2])
    c, tc = pool.alloc(2)
    assert sorted(c.tolist()) == sorted(a[:2].tolist()) and np.all(tc == 2)
    pool.reallocate(int(b[0]))
    assert pool.tags[b[0]] == 2


def test_allocate_batch_shapes():
    pool = I.PagePool(100, seed=0)
    bt = I.allocate_batch(pool, [1, 16, 17, 33], 16)
    assert bt.page_table.shape == (4, 3)
    assert (bt.page_table[0, 1:] == -1).all() and (bt.page_table[3] >= 0).all()
    assert bt.expected_tags[3].tolist() == [1, 1, 1]


def test_workload_pool_sizes():
    w = I.WORKLOADS["gqa8_16k_b64"]
    assert w.pool_pages == 16384
    assert I.sweep_workload(32, 2).pool_pages == 8192
    assert I.WORKLOADS["gqa8_256k_b4"].group == 8


def test_fixed_pool_budget_is_never_enlarged():
    with pytest.raises(I.PoolExhausted):
        I.make_decode_inputs(I.Workload("w", 3, 2, 2, 64, 16, 64, 64, pool_pages=11), 0)
    inp = I.make_decode_inputs(I.Workload("w", 3, 2, 2, 64, 16, 64, 64, pool_pages=12), 0)
    assert inp.num_pages == 12 and inp.pool.free_pages == 0


def _scores(inp, b=0):
    """fp64 scores [Hq][L] of request b from the bf16 inputs (no quantisation)."""
    w = inp.workload
    q = inp.q[b].float().double().numpy()                       # [Hq][D]
    k = inp.k_tokens[b].float().double().numpy()                # [T][Hkv][D]
    G = w.group
    return np.stack([k[:, h // G, :] @ q[h] for h in range(w.q_heads)]) / np.sqrt(w.head_dim)


def test_needle_recipe_is_the_intended_regime():
    """The needle recipe (drawn on the CPU here; the GPU tests draw it on the
    device): needles score needle_gap above a flat background for every head
    of the group, and the background's weights lie where fp16 has no normal
    numbers, so that weights rounded to fp16 miss the parity tolerance on the
    biased channels while a bf16 high + low pair of each weight meets it."""
    L = 262144
    w = I.Workload("needle", 1, 8, 1, 128, 64, L, L, needle_gap=17.6, v_bias=4.0)
    inp = I.make_device_decode_inputs(w, 1200, "cpu")
    s = _scores(inp)
    needles = np.arange(0, I.NEEDLE_SPAN, I.NEEDLE_EVERY)
    bg = np.ones(L, bool)
    bg[needles] = False
    gap = s[:, needles].min(axis=1) - s[:, bg].max(axis=1)
    assert np.all(gap > 17.3) and np.all(s[:, needles].max(axis=1) - s[:, needles].min(axis=1) < 0.1)
    assert np.all(s[:, bg].max(axis=1) - s[:, bg].min(axis=1) < 0.5)
    v = inp.v_tokens[0, :, 0, :].float().double().numpy()      # [L][D]
    for h in range(w.q_heads):
        p = np.exp(s[h] - s[h].max())
        ref = (p @ v) / p.sum()
        p16 = p.astype(np.float16).astype(np.float64)
        got16 = (p16 @ v) / p.sum()
        hi = I.bf16_bits_to_f32(I.f32_to_bf16_bits(p.astype(np.float32))).astype(np.float64)
        lo = I.bf16_bits_to_f32(I.f32_to_bf16_bits((p - hi).astype(np.float32))).astype(np.float64)
        got_b = ((hi + lo) @ v) / p.sum()
        tol = 2e-3 + 1e-2 * np.abs(ref)
        assert np.any(np.abs(got16 - ref) > tol), "fp16 weights would pass: the recipe is too weak"
        assert np.all(np.abs(got_b - ref) < 1e-5)


def test_scaled_and_biased_recipes():
    """K/V data scaled by 2^e is the unscaled draw times 2^e exactly (so are
    the scales); the V bias lands on the even head dims; q_mult scales q."""
    base = I.Workload("r", 2, 8, 2, 128, 64, 300, 300, pool_factor=1.25, v_bias=4.0)
    a = I.make_device_decode_inputs(base, 5, "cpu")
    b = I.make_device_decode_inputs(I.scaled(base, k_log2=20, v_log2=-20), 5, "cpu")
    assert torch.equal(b.k_tokens.float(), a.k_tokens.float() * 2.0 ** 20)
    assert torch.equal(b.v_tokens.float(), a.v_tokens.float() * 2.0 ** -20)
    assert np.array_equal(b.k_scale, a.k_scale * np.float32(2.0 ** 20))
    assert np.array_equal(b.v_scale, a.v_scale * np.float32(2.0 ** -20))
    v = a.v_tokens.float()
    assert abs(float(v[..., 0::2].mean()) - 4.0) < 0.05 and abs(float(v[..., 1::2].mean())) < 0.05
    c = I.make_device_decode_inputs(I.scaled(base, q_mult=16.0), 5, "cpu")
    assert 14.0 < float(c.q.float().std()) < 18.0
    # the plain recipe is unchanged by the new fields' defaults
    d = I.make_device_decode_inputs(I.Workload("r", 2, 8, 2, 128, 64, 300, 300, pool_factor=1.25), 5, "cpu")
    assert abs(float(d.q.float().std()) - 1.0) < 0.1
