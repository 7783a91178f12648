"""The entry points under HIP graph capture.  Every call launches kernels on
the caller's stream and nothing else (no allocation, no memset, no host
synchronisation), so a caller may capture a decode step, a hand-off or an
INT4 GEMV into a graph.  Each captured sequence is replayed several times,
with eager work on the same device between the replays, and every replay's
outputs must equal the eager run's bit for bit (the kernels are
deterministic)."""
import math

import numpy as np
import pytest
import torch

from paged_attention_fp8_amd import harness as H
from paged_attention_fp8_amd import inputs as I
from paged_attention_fp8_amd import ops

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def say(*a):
    print(*a, flush=True)


def capture(fn):
    """fn captured into a graph, after one warm-up on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def check_replays(g, outputs, want, scramble, eager_between):
    for r in range(REPLAYS):
        scramble()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("out", "lse", "status"), outputs, want):
            assert torch.equal(got, ref), (r, name)
        eager_between()
        torch.cuda.synchronize()


@pytest.mark.parametrize("kv_dtype,splits", [(ops.KV_FP8_E4M3, 4), (ops.KV_FP8_E4M3, 1), (ops.KV_BF16, 2),
                                             (ops.KV_FP8_E4M3, -8)])
def test_decode_step_replays(kv_dtype, splits):
    """Check + append + attention (+ combine when split; splits < 0: the
    balanced partition) captured as one graph."""
    say(f"graph: decode step dtype={kv_dtype} S={splits}")
    w = I.Workload("graph_step", 3, 16, 4, 128, 64, 300, 900, pool_factor=1.3, stale_requests=1)
    inp = I.make_decode_inputs(w, 31)
    step = H.build_step(inp, kv_dtype, DEV)
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    sm = 1.0 / math.sqrt(D)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    status = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = torch.empty(max(ops.workspace_bytes(B, Hq, D, splits), 16), dtype=torch.uint8, device=DEV)

    def one():
        stat = ops.page_tag_check(step.batch, w.page_size, step.page_tags, step.expected_tags, out=status)
        b = step.batch.with_status(stat)
        ops.kv_quant_append(step.cache, b, step.k_new, step.v_new)
        ops.paged_decode_attn(step.cache, b, step.q, sm, splits, ws, out, lse)

    one()
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone(), status.clone())
    assert int((want[2] != 0).sum()) == 1          # the stale request is aborted in the graph too
    g = capture(one)
    other_out = torch.empty_like(out)

    def scramble():
        out.fill_(3.0)
        lse.fill_(3.0)
        status.fill_(-1)
        ws.fill_(0x55)

    def eager_between():   # the same kernels, eagerly, into other buffers
        ops.paged_decode_attn(step.cache, step.batch.with_status(status), step.q, sm, 1, None,
                              other_out, None, return_lse=False)

    check_replays(g, (out, lse, status), want, scramble, eager_between)


def test_fill_and_int4_replay():
    """kv_quant_fill (partial tiles included) and int4_gemv at 1 and 5 rows."""
    say("graph: fill + int4 gemv")
    w = I.Workload("graph_fill", 2, 8, 2, 128, 64, 200, 200, pool_factor=1.0)
    inp = I.make_decode_inputs(w, 32)
    cache = H.new_cache(w, inp.num_pages, ops.KV_FP8_E4M3, DEV, inp.k_scale, inp.v_scale)
    batch, _, _ = H.upload_batch(inp.batch, inp.pool, DEV)
    T = 150
    k = H.bf16_tensor(np.stack([inp.k_tokens[b][:T] for b in range(2)]), DEV)
    v = H.bf16_tensor(np.stack([inp.v_tokens[b][:T] for b in range(2)]), DEV)
    start = torch.tensor([5, 40], dtype=torch.int32, device=DEV)
    count = torch.tensor([T, T - 33], dtype=torch.int32, device=DEV)
    g = np.random.default_rng(33)
    N, K = 64, 1024
    wq = torch.from_numpy(g.integers(0, 256, N * K // 2).astype(np.uint8)).to(DEV)
    sc = torch.from_numpy(I.f32_to_bf16_bits((g.random((K // 128, N)) * 0.05 + 1e-3).astype(np.float32))
                          .view(np.int16)).to(DEV).view(torch.bfloat16)
    x1 = torch.randn((1, K), device=DEV).to(torch.bfloat16)
    x5 = torch.randn((5, K), device=DEV).to(torch.bfloat16)
    y1 = torch.empty((1, N), dtype=torch.float32, device=DEV)
    y5 = torch.empty((5, N), dtype=torch.float32, device=DEV)

    def seq():
        ops.kv_quant_fill(cache, batch, start, count, k, v)
        ops.int4_gemv(x1, wq, sc, N, K, out=y1)
        ops.int4_gemv(x5, wq, sc, N, K, out=y5)

    seq()
    torch.cuda.synchronize()
    want = (cache.k_pool.clone(), cache.v_pool.clone(), y1.clone(), y5.clone())
    gr = capture(seq)
    for r in range(REPLAYS):
        H.poison_(cache)
        y1.fill_(3.0)
        y5.fill_(3.0)
        gr.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("k_pool", "v_pool", "y1", "y5"), (cache.k_pool, cache.v_pool, y1, y5), want):
            assert torch.equal(got, ref), (r, name)
        ops.int4_gemv(x5, wq, sc, N, K)      # eager work between replays
        torch.cuda.synchronize()
