"""paged_decode_attn_fp8_noalloc: the entry point for callers that cannot
allocate.  Its outputs must equal paged_decode_attn_fp8's (caller workspace,
same split count) bit for bit, on two calls in a row -- the second on a
smaller batch, so that the scratch still holds the first call's partials --
for uniform splits, the library default and the balanced partition; and
against the oracle's tolerance."""
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

BIG = I.Workload("noalloc_big", 6, 32, 4, 128, 64, 700, 4000, pool_factor=1.3, stale_requests=1)
SMALL = I.Workload("noalloc_small", 2, 16, 2, 128, 16, 100, 900, pool_factor=1.5)


def _same(a, b):
    return torch.equal(a, b) or np.array_equal(a.cpu().numpy(), b.cpu().numpy(), equal_nan=True)


@pytest.mark.parametrize("splits", [4, 0, ops.BALANCED], ids=["S4", "default", "balanced"])
def test_noalloc_equals_workspace_call_twice(splits):
    for w, seed in ((BIG, 501), (SMALL, 502)):      # second call: fewer requests, heads, pages
        print(f"noalloc: {w.name} splits={splits}", flush=True)
        inp = I.make_decode_inputs(w, seed)
        step = H.build_step(inp, ops.KV_FP8_E4M3, DEV, poison=True)
        sm = 1.0 / math.sqrt(w.head_dim)
        status = ops.page_tag_check(step.batch, w.page_size, step.page_tags, step.expected_tags)
        b = step.batch.with_status(status)
        ops.kv_quant_append(step.cache, b, step.k_new, step.v_new)
        ref_o, ref_l = ops.paged_decode_attn(step.cache, b, step.q, sm, splits)
        out, lse = ops.paged_decode_attn_noalloc(step.cache, b, step.q, sm, splits,
                                                 lse=torch.empty_like(ref_l))
        torch.cuda.synchronize()
        assert _same(out, ref_o) and _same(lse, ref_l)
        st = status.cpu().numpy()
        pool = oracle_pool(inp, oracle.KV_FP8, poison=True, append=False)
        oracle.kv_append(pool, inp.batch.page_table, inp.batch.context_lens, inp.k_new(), inp.v_new(),
                         inp.k_scale, inp.v_scale, status=st)
        ro, rl = oracle.paged_attention(pool, inp.q, inp.batch.page_table, inp.batch.context_lens, sm,
                                        inp.k_scale, inp.v_scale, status=st)
        live = st == 0
        ok1, ma, _ = allclose_report(out.cpu().numpy()[live], ro[live])
        ok2, la, _ = allclose_report(lse.cpu().numpy()[live], rl[live])
        print(f"  bitwise equal to the workspace call; oracle max_abs out {ma:.2e} lse {la:.2e}", flush=True)
        assert ok1 and ok2
        assert np.all(out.cpu().numpy()[~live] == 0)


def test_noalloc_rejects_partials_beyond_its_scratch():
    """16 requests x 64 query heads x 64 splits of 128-dim partials need
    33.8 MB: refused before anything is launched (the data is never read)."""
    B, Hq, Hkv, D, P = 16, 64, 8, 128, 64
    ones = torch.ones(Hkv, dtype=torch.float32, device=DEV)
    cache = ops.PagedKVCache.allocate(16, Hkv, P, D, ops.KV_FP8_E4M3, DEV, ones, ones)
    batch = ops.DecodeBatch(torch.zeros((B, 64), dtype=torch.int32, device=DEV),
                            torch.full((B,), 64 * P, dtype=torch.int32, device=DEV))
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    assert ops.workspace_bytes(B, Hq, D, 64) > ops.noalloc_scratch_bytes()
    with pytest.raises(ops.Pafp8Error, match="scratch"):
        ops.paged_decode_attn_noalloc(cache, batch, q, 0.1, 64)
