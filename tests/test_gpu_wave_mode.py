"""Wave-per-split mode: when a launch has at least one split per wave slot of
the GPU (4 x num_cus split units), every wave takes whole splits of one
(request, KV head) and writes their partial rows itself, and the combine
merges them.  The library picks the mode from the launch size; these batches
are sized to select it on 256 CUs (48 requests x 8 KV heads x 16 or 7
splits: 6 or 2 splits per wave, with a shorter last chunk; and one query
head per KV head, 12 requests x 32 KV heads x 16 or 3 splits: two splits or
one per wave), with ragged lengths
(requests that end inside a split, splits past a request's end), one aborted
request, both pool types; every output against the oracle, and the pools
byte for byte.  The same requests through the work-group mode (one request
per launch) agree within the tolerance too."""
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


GROUPS = {"g8": (48, 64, 8), "g1": (12, 32, 32)}   # requests, query heads, KV heads


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("group,splits", [("g8", 16), ("g8", 7), ("g1", 16), ("g1", 3)])
def test_wave_mode_matches_oracle(kv_dtype, group, splits):
    B, Hq, Hkv = GROUPS[group]
    w = I.Workload("wavemode", B, Hq, Hkv, 128, 64, 300, 4096, pool_factor=1.2, stale_requests=1)
    print(f"wave mode: dtype={kv_dtype} {group} splits={splits}", flush=True)
    lengths = I.context_lengths(w, 901)
    lengths[7] = 4096                                  # max_pages_per_req = 64
    inp = I.make_decode_inputs(w, 901, lengths=lengths)
    lens = inp.batch.context_lens.copy()
    step = H.build_step(inp, kv_dtype, DEV, poison=True)
    sm = 1.0 / math.sqrt(w.head_dim)
    status = ops.page_tag_check(step.batch, w.page_size, step.page_tags, step.expected_tags)
    b_all = step.batch.with_status(status)
    ops.kv_quant_append(step.cache, b_all, step.k_new, step.v_new)
    out, lse = ops.paged_decode_attn(step.cache, b_all, step.q, sm, splits)
    torch.cuda.synchronize()
    st = status.cpu().numpy()
    assert int((st != 0).sum()) == 1
    ks = inp.k_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    vs = inp.v_scale if kv_dtype == ops.KV_FP8_E4M3 else None
    pool = oracle_pool(inp, kv_dtype, poison=True, append=False)
    oracle.kv_append(pool, inp.batch.page_table, lens, inp.k_new(), inp.v_new(), ks, vs, status=st)
    ro, rl = oracle.paged_attention(pool, inp.q, inp.batch.page_table, lens, sm, ks, vs, status=st)
    live = st == 0
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    ok1, ma, _ = allclose_report(o[live], ro[live])
    ok2, la, _ = allclose_report(l[live], rl[live])
    print(f"  every output: out max_abs {ma:.2e}, lse max_abs {la:.2e}", flush=True)
    assert ok1 and ok2
    assert np.all(o[~live] == 0) and np.all(np.isneginf(l[~live]))
    for b in (int(np.argmin(lens)), int(np.argmax(lens)), 5):
        one = ops.DecodeBatch(step.batch.page_table[b:b + 1].contiguous(),
                              step.batch.context_lens[b:b + 1].contiguous(), status[b:b + 1].contiguous())
        o1, l1 = ops.paged_decode_attn(step.cache, one, step.q[b:b + 1].contiguous(), sm, splits)
        torch.cuda.synchronize()
        o1, l1 = o1.cpu().numpy(), l1.cpu().numpy()
        if st[b] != 0:   # the aborted request: fixed outputs
            assert np.all(o1 == 0) and np.all(np.isneginf(l1)), f"aborted request {b} alone"
            continue
        ok1, ma, _ = allclose_report(o1, ro[b:b + 1])
        ok2, la, _ = allclose_report(l1, rl[b:b + 1])
        assert ok1 and ok2, f"request {b} alone: out {ma}, lse {la}"
