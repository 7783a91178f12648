"""PreparedCall: the tag check and the attention (plain and with the append
in its launch) marshalled once and run many times give, bit for bit, what
the per-call entry points give -- also after the inputs' contents change in
place between runs, and on an explicitly given stream."""
import math

import numpy as np
import pytest
import torch

from paged_attention_fp8_amd import harness as H
from paged_attention_fp8_amd import inputs as I
from paged_attention_fp8_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _same(a, b):
    return np.array_equal(a.cpu().numpy(), b.cpu().numpy(), equal_nan=True)


@pytest.mark.parametrize("splits", [1, 4, ops.BALANCED], ids=["S1", "S4", "balanced"])
def test_prepared_equals_eager(splits):
    print(f"prepared calls: splits={splits}", flush=True)
    w = I.Workload("prep_gqa8", 3, 16, 2, 128, 64, 300, 1500, pool_factor=1.3, stale_requests=1)
    inp = I.make_decode_inputs(w, 91)
    sm = 1.0 / math.sqrt(w.head_dim)
    a = H.build_step(inp, ops.KV_FP8_E4M3, DEV, poison=True)
    b = H.build_step(inp, ops.KV_FP8_E4M3, DEV, poison=True)
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    status = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    chk = ops.prepare_page_tag_check(b.batch, w.page_size, b.page_tags, b.expected_tags, status)
    att = ops.prepare_paged_decode_attn(b.cache, b.batch.with_status(status), b.q, sm, splits,
                                        out=out, lse=lse, k_new=b.k_new, v_new=b.v_new)
    side = torch.cuda.Stream()
    for rnd in range(3):
        if rnd == 2:   # new query contents, same tensors
            for st in (a, b):
                st.q.copy_(torch.flip(st.q, dims=[1]))
        oa, la, sa = H.decode_step(a, sm, splits, append_in_attention=True)
        if rnd == 1:
            side.wait_stream(torch.cuda.current_stream())
            chk.run(side.cuda_stream)
            ob, lb = att.run(side.cuda_stream)
            torch.cuda.current_stream().wait_stream(side)
        else:
            chk.run()
            ob, lb = att.run()
        torch.cuda.synchronize()
        assert ob is out and lb is lse
        assert _same(sa, status) and int((status != 0).sum()) == 1, rnd
        assert _same(oa, out) and _same(la, lse), rnd
        assert _same(a.cache.k_pool, b.cache.k_pool) and _same(a.cache.v_pool, b.cache.v_pool), rnd


def test_prepared_errors_are_raised():
    """A prepared call checks its arguments when it is prepared, and a launch
    error comes back from run() as Pafp8Error."""
    w = I.Workload("prep_err", 2, 16, 2, 128, 64, 100, 300, pool_factor=1.5)
    inp = I.make_decode_inputs(w, 92)
    st = H.build_step(inp, ops.KV_FP8_E4M3, DEV)
    with pytest.raises(ValueError, match="shape"):
        ops.prepare_paged_decode_attn(st.cache, st.batch, st.q[:1].contiguous(), 0.1, 1)
    bad = ops.prepare_paged_decode_attn(st.cache, st.batch, st.q, -1.0, 1)   # checked by the library
    with pytest.raises(ops.Pafp8Error, match="sm_scale"):
        bad.run()
