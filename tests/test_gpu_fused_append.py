"""paged_decode_attn_{fp8,bf16}_append: the append taken into the attention
launch must leave the same pool bytes and give bitwise the same out and lse
as kv_quant_append followed by the attention call (same kernels, same data),
for uniform splits and the balanced partition, with stale requests, and under
graph capture (a replay appends the same token again)."""
import math

import numpy as np
import pytest
import torch

from paged_attention_fp8_amd import harness as H
from paged_attention_fp8_amd import inputs as I
from paged_attention_fp8_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    I.Workload("mha_d64_p16", 3, 4, 4, 64, 16, 1, 300, pool_factor=1.5),
    I.Workload("gqa4_d128_p16", 3, 16, 4, 128, 16, 250, 1100, pool_factor=1.3),
    I.Workload("gqa8_d128_p64", 4, 16, 2, 128, 64, 1, 1500, pool_factor=1.3),
    I.Workload("gqa16_d64_p32", 2, 32, 2, 64, 32, 300, 900, pool_factor=1.3),
    I.Workload("gqa5_d128_p256", 2, 10, 2, 128, 256, 700, 1300, pool_factor=1.3),
]


def _bits(t, kv_dtype):
    t = t.cpu()
    return t.view(torch.int16).numpy() if kv_dtype == ops.KV_BF16 else t.numpy()


def _same(a, b):
    return np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("splits", [1, 3, ops.BALANCED], ids=["S1", "S3", "balanced"])
@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_fused_equals_separate(w, kv_dtype, splits):
    print(f"fused append: {w.name} dtype={kv_dtype} splits={splits}", flush=True)
    inp = I.make_decode_inputs(I.scaled(w, stale_requests=1 if w.batch > 2 else 0), 41)
    sm = 1.0 / math.sqrt(w.head_dim)
    a = H.build_step(inp, kv_dtype, DEV, poison=True)
    b = H.build_step(inp, kv_dtype, DEV, poison=True)
    oa, la, sa = H.decode_step(a, sm, splits)
    ob, lb, sb = H.decode_step(b, sm, splits, append_in_attention=True)
    torch.cuda.synchronize()
    assert torch.equal(sa, sb)
    if w.batch > 2:
        assert int((sa != 0).sum()) == 1           # the stale request is aborted either way
    assert _same(_bits(a.cache.k_pool, kv_dtype), _bits(b.cache.k_pool, kv_dtype))
    assert _same(_bits(a.cache.v_pool, kv_dtype), _bits(b.cache.v_pool, kv_dtype))
    assert _same(oa.cpu().numpy(), ob.cpu().numpy()) and _same(la.cpu().numpy(), lb.cpu().numpy())


def test_fused_without_tracker_and_bad_inputs():
    """No status array: a page id outside the pool and a length past the table
    give NaN rows and no write, length 0 gives 0 / -inf, exactly as the
    separate calls."""
    w = CASES[2]
    inp = I.make_decode_inputs(w, 42)
    steps = [H.build_step(inp, ops.KV_FP8_E4M3, DEV) for _ in range(2)]
    res = []
    for k, st in enumerate(steps):
        pt = st.batch.page_table.clone()
        lens = st.batch.context_lens.clone()
        pt[0, 0] = st.cache.num_pages + 3
        lens[1] = 0
        lens[2] = pt.shape[1] * w.page_size + 1
        batch = ops.DecodeBatch(pt, lens)
        if k == 0:
            ops.kv_quant_append(st.cache, batch, st.k_new, st.v_new)
            o, l = ops.paged_decode_attn(st.cache, batch, st.q, 0.09, 2)
        else:
            o, l = ops.paged_decode_attn(st.cache, batch, st.q, 0.09, 2, k_new=st.k_new, v_new=st.v_new)
        torch.cuda.synchronize()
        res.append((o.cpu().numpy(), l.cpu().numpy(), st.cache.k_pool.cpu().numpy(),
                    st.cache.v_pool.cpu().numpy()))
    for x, y in zip(res[0], res[1]):
        assert _same(x, y)
    o = res[1][0]
    assert np.all(np.isnan(o[0])) and np.all(np.isnan(o[2])) and np.all(o[1] == 0)


def test_fused_step_under_graph_capture():
    """check + fused append-attention captured once and replayed: every replay
    writes the same token and gives the eager outputs bit for bit."""
    w = CASES[1]
    inp = I.make_decode_inputs(w, 43)
    st = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    status = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = torch.empty(max(ops.workspace_bytes(B, Hq, D, 3), 16), dtype=torch.uint8, device=DEV)

    def one():
        s = ops.page_tag_check(st.batch, w.page_size, st.page_tags, st.expected_tags, out=status)
        ops.paged_decode_attn(st.cache, st.batch.with_status(s), st.q, 0.1, 3, ws, out, lse,
                              k_new=st.k_new, v_new=st.v_new)

    one()
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone(), st.cache.k_pool.clone(), st.cache.v_pool.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    for r in range(3):
        out.fill_(3.0)
        lse.fill_(3.0)
        g.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out, lse, st.cache.k_pool, st.cache.v_pool), want):
            assert torch.equal(got, ref), r
