"""Parity at the full sizes of the measured workloads, in the launch
configuration bench.py times (library-default split count unless the
workload fixes one), on sampled requests the oracle computes one by one.

Workloads (named by what they are):
  tiny_mha_d64_256    1 request, 4/4 heads, d64, 256 tokens, 16-token pages (all outputs)
  gqa4_4k_outliers    8 requests, 32/8 heads, d128, 4096 tokens, 16-token pages,
                      1% outliers x20 saturating (all outputs)
  gqa8_ragged_32k     32 requests, 64/8 heads, d128, 1024..32768 tokens, 64-token pages,
                      fragmented pool; e4m3 and the identical-source bf16 cache, default
                      splits and the balanced partition (3 sampled requests)
  gqa8_16k_b64        64 requests x 16384 tokens, 2 GiB pool (2 sampled requests); the
                      bf16 twin at 32 requests (1 sampled request)
  gqa8_256k_b4        4 requests x 262144 tokens, 64 splits, one stale request that must
                      be aborted (1 sampled request, one KV group)
  handoff_8k_b8       kv_quant_fill of 8 prompts x 8192 tokens into e4m3 pages (whole
                      pools byte for byte)
For sampled requests the pool pages they own must equal the oracle's byte for
byte, and every output within 2e-3 abs + 1e-2 rel.
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


def say(*a):
    print(*a, flush=True)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sampled_oracle(inp, kv_dtype, reqs, heads=None):
    """Oracle pool holding just the sampled requests (quantised by the oracle
    from the same bf16 source), and the oracle outputs for them."""
    w = inp.workload
    fill = H.FP8_NAN_CODE if kv_dtype == oracle.KV_FP8 else H.BF16_NAN_BITS  # as run_step
    pool = oracle.Pool(kv_dtype, inp.num_pages, w.kv_heads, w.page_size, w.head_dim, fill=fill)
    table = inp.batch.page_table
    lens = inp.batch.context_lens
    ks = inp.k_scale if kv_dtype == oracle.KV_FP8 else None
    vs = inp.v_scale if kv_dtype == oracle.KV_FP8 else None
    for b in reqs:
        L = int(lens[b])
        k = host_bits(inp.k_tokens[b, :L])[None]
        v = host_bits(inp.v_tokens[b, :L])[None]
        oracle.kv_write(pool, table[b:b + 1], np.zeros(1, np.int32), np.array([L], np.int32),
                        k, v, ks, vs)
    q = host_bits(inp.q)
    res = {}
    sm = 1.0 / math.sqrt(w.head_dim)
    if heads is None:
        o, l = oracle.paged_attention(pool, q[reqs], table[reqs], lens[reqs], sm, ks, vs)
        for i, b in enumerate(reqs):
            for h in range(w.q_heads):
                res[b, h] = (o[i, h], l[i, h])
    else:
        for b in reqs:
            for h in heads:
                res[b, h] = oracle.attention_range(pool, q, table, b, h, 0, int(lens[b]), sm,
                                                   ks, vs)
    return pool, res


def check_sampled(step, inp, kv_dtype, out, lse, reqs, heads=None):
    pool, res = sampled_oracle(inp, kv_dtype, reqs, heads)
    gk, gv = step.cache.k_pool.cpu(), step.cache.v_pool.cpu()
    if kv_dtype == ops.KV_BF16:
        gk = gk.view(torch.int16).numpy().view(np.uint16)
        gv = gv.view(torch.int16).numpy().view(np.uint16)
    else:
        gk, gv = gk.numpy(), gv.numpy()
    for b in reqs:
        pages = inp.batch.page_table[b][: I.pages_needed(inp.batch.context_lens[b], inp.workload.page_size)]
        assert np.array_equal(gk[pages], pool.k[pages]), f"K pages of request {b} differ"
        assert np.array_equal(gv[pages], pool.v[pages]), f"V pages of request {b} differ"
    ro = np.stack([res[k][0] for k in sorted(res)])
    rl = np.array([res[k][1] for k in sorted(res)])
    go = np.stack([out[b, h] for (b, h) in sorted(res)])
    gl = np.array([lse[b, h] for (b, h) in sorted(res)])
    ok1, ma, mr = allclose_report(go, ro)
    ok2, la, lr = allclose_report(gl, rl)
    say(f"  sampled {len(res)} rows: out max_abs={ma:.3e} max_rel={mr:.3e}, lse max_abs={la:.3e}")
    assert ok1 and ok2


def run_step(inp, kv_dtype, splits=0):
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(inp.workload.head_dim)
    out, lse, status = H.decode_step(step, sm, splits)
    torch.cuda.synchronize()
    return step, out.cpu().numpy(), lse.cpu().numpy(), status.cpu().numpy()


@pytest.mark.parametrize("balanced", [False, True], ids=["splits", "balanced"])
@pytest.mark.parametrize("name", ["tiny_mha_d64_256", "gqa4_4k_outliers"])
def test_small_workloads_all_outputs(name, balanced):
    """Every output, with the workload's split count and with the balanced
    partition (for the single tiny request every range cuts it)."""
    w = I.WORKLOADS[name]
    say(f"workload {name} balanced={balanced}")
    inp = I.make_decode_inputs(w, 1001)
    step, out, lse, status = run_step(inp, ops.KV_FP8_E4M3, ops.BALANCED if balanced else w.num_splits)
    assert np.all(status == 0)
    ref = oracle_pool(inp, oracle.KV_FP8, poison=True)
    assert np.array_equal(step.cache.k_pool.cpu().numpy(), ref.k)
    assert np.array_equal(step.cache.v_pool.cpu().numpy(), ref.v)
    if w.outlier_frac:
        # the outliers really saturate: some codes are +-448
        assert np.isin(ref.k, [0x7E, 0xFE]).any()
    ro, rl = oracle.paged_attention(ref, inp.q, inp.batch.page_table, inp.batch.context_lens,
                                    1.0 / math.sqrt(w.head_dim), inp.k_scale, inp.v_scale)
    ok1, ma, mr = allclose_report(out, ro)
    ok2, la, _ = allclose_report(lse, rl)
    say(f"  all outputs: out max_abs={ma:.3e} max_rel={mr:.3e}, lse max_abs={la:.3e}")
    assert ok1 and ok2


@pytest.mark.parametrize("splits", [0, ops.BALANCED], ids=["default", "balanced"])
@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
def test_ragged_32k(kv_dtype, splits):
    """Default splits and the balanced partition, whose ranges cut the longest
    requests (sampled: the shortest, the longest and request 7)."""
    w = I.WORKLOADS["gqa8_ragged_32k"]
    say(f"workload {w.name} dtype={kv_dtype} splits={splits}")
    inp = I.make_device_decode_inputs(w, 1002, DEV)
    step, out, lse, status = run_step(inp, kv_dtype, splits)
    assert np.all(status == 0)
    lens = inp.batch.context_lens
    reqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 7})
    check_sampled(step, inp, kv_dtype, out, lse, reqs)


def test_concurrency_point_b64():
    w = I.WORKLOADS["gqa8_16k_b64"]
    say(f"workload {w.name}")
    inp = I.make_device_decode_inputs(w, 1003, DEV)
    step, out, lse, status = run_step(inp, ops.KV_FP8_E4M3)
    assert np.all(status == 0)
    check_sampled(step, inp, ops.KV_FP8_E4M3, out, lse, [0, 63])


def test_bf16_twin_b32_and_capacity():
    w = I.sweep_workload(32, 2)
    say(f"workload {w.name} bf16")
    assert w.pool_pages == 8192
    with pytest.raises(I.PoolExhausted):
        I.make_device_decode_inputs(I.sweep_workload(33, 2), 1004, DEV)
    inp = I.make_device_decode_inputs(w, 1004, DEV)
    step, out, lse, status = run_step(inp, ops.KV_BF16)
    assert np.all(status == 0)
    check_sampled(step, inp, ops.KV_BF16, out, lse, [5])


def test_long_context_256k_with_stale_request():
    w = I.WORKLOADS["gqa8_256k_b4"]
    say(f"workload {w.name}")
    inp = I.make_device_decode_inputs(w, 1005, DEV)
    assert len(inp.stale) == 1
    step, out, lse, status = run_step(inp, ops.KV_FP8_E4M3, w.num_splits)
    bad = inp.stale[0]
    want = np.zeros(4, np.int32)
    want[bad] = oracle.REQ_TAG_MISMATCH
    assert np.array_equal(status, want)
    ref_status = oracle.page_tag_check(inp.batch.page_table, inp.batch.context_lens,
                                       inp.batch.expected_tags, inp.pool.tags, w.page_size)
    assert np.array_equal(status, ref_status)
    assert np.all(out[bad] == 0) and np.all(np.isneginf(lse[bad]))
    good = [b for b in range(4) if b != bad]
    check_sampled(step, inp, ops.KV_FP8_E4M3, out, lse, [good[0]], heads=range(8, 16))


def test_prefill_handoff_full_size_pools_bit_exact():
    """The prefill-to-decode hand-off the bench times (8 prompts x 8192 bf16
    tokens, 8 KV heads, d128, 64-token pages -> e4m3; one kv_quant_fill
    launch): both pools byte for byte against the oracle.  A second fill of
    the same sources at ragged starts and counts (partial tiles and groups in
    every request) into a fresh pool, likewise."""
    w = I.Workload("handoff_8k_b8", 8, 64, 8, 128, 64, 8192, 8192, pool_factor=1.0)
    say(f"workload {w.name}")
    inp = I.make_device_decode_inputs(w, 1006, DEV)
    B, T = w.batch, w.max_len
    k, v = inp.k_tokens[:, :T].contiguous(), inp.v_tokens[:, :T].contiguous()
    kh, vh = host_bits(k), host_bits(v)
    dbatch, _, _ = H.upload_batch(inp.batch, inp.pool, DEV)
    g = np.random.default_rng(6)
    cases = [(np.zeros(B, np.int32), np.full(B, T, np.int32))]
    cases.append((g.integers(0, 200, B).astype(np.int32), g.integers(T - 700, T - 200, B).astype(np.int32)))
    for start, count in cases:
        cache = H.new_cache(w, inp.num_pages, ops.KV_FP8_E4M3, DEV, inp.k_scale, inp.v_scale)
        ops.kv_quant_fill(cache, dbatch, torch.from_numpy(start).to(DEV), torch.from_numpy(count).to(DEV), k, v)
        ref = oracle.Pool(oracle.KV_FP8, inp.num_pages, w.kv_heads, w.page_size, w.head_dim,
                          fill=H.FP8_NAN_CODE)
        oracle.kv_write(ref, inp.batch.page_table, start, count, kh, vh, inp.k_scale, inp.v_scale)
        assert np.array_equal(cache.k_pool.cpu().numpy(), ref.k)
        assert np.array_equal(cache.v_pool.cpu().numpy(), ref.v)
        say(f"  starts {start[:3]}..., counts {count[:3]}...: pools bit-exact")
        del cache, ref
        torch.cuda.empty_cache()
