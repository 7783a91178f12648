"""Benchmark of the decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-extras] [--only NAME[,NAME]] [--copy-calibration]
                    [--summarize-counters ...]

One step = one pass of the path over one batch: the batched page-tag check,
the quantise-on-append of this step's token for every request, and e4m3 paged
decode attention (with its split-K combine when the library splits).  The workload is the concurrency point the target is quoted
on: 64 requests of 16,384 tokens, 64 query heads on 8 KV heads, head_dim 128,
64-token pages, in a 2 GiB pool that holds exactly 64 e4m3 requests (or 32
bf16 ones).  Inputs are seeded synthetic data drawn on the GPU and resident in
HBM before timing.

Prints one JSON line.  value = attention tokens/s (one decode token per
request through one attention layer per step).  roofline.achieved is the
algorithmic bytes of one attention launch divided by its mean duration,
measured with HIP events on the launch stream over the timed steps.  Beside
it: the tag-check overhead against the no-op tracker (separate pass, and
inside the append launch), the append inside the attention launch (64
requests and one), the bf16 twin (32 requests: the same KV bytes), and the
extras -- the concurrency sweep of the pages' decode table (1/8/16/32/64
requests, e4m3 and bf16, each step after a 1 GiB read of other memory so
that no point runs out of the MALL), the 4k-token / 16-token-page workload,
one query head per KV head (8 x 16k tokens, 32 heads),
the long-context point (4 requests of 262,144 tokens in 64 splits: check
overhead, and the batch with one stale request), the prefill-to-decode
hand-off (kv_quant_fill of 8 prompts of 8,192 tokens), a continuous decode
loop with admission under the same 2 GiB budget (e4m3 vs bf16), INT4 weight
streaming (int4_gemv over 940 MB of int4 weights at 1-64 rows), and the
ragged batch (32 requests of 1k-32k tokens) on e4m3 and bf16 caches from one
bf16 source.  Beside each HBM-bound point stands the bare stream of its bytes
(pafp8_stream_read, or pafp8_stream_read_write for the hand-off), launched and
timed the same way: what the memory system delivers at that size.  --only
runs named extras alone (for profiling one workload).
cpu_baseline times the CPU oracle on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
COUNTERS_SUMMARY = os.path.join(ROOT, "profiles", "decode_attn_e4m3_gqa8_16k_b64_counters.md")
COPY_BYTES = 1 << 30
FLUSH_BYTES = 1 << 30
SEED = 1003
METRIC = "decode attention tokens/s and achieved HBM GB/s (% of peak), FP8 vs BF16 KV"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# The driver clears device memory that is allocated or released, in the
# background: for a few seconds after a multi-GiB pool comes or goes, kernels
# share HBM with that clearing (measured here: after a 2 GiB release the next
# attention calls run ~4% slower, and within 5 s they are back to normal).
# Every timed section therefore starts once the device has been quiet for
# SETTLE_S seconds since the last segment was allocated or freed.
SETTLE_S = 5.0
_settled_at = None


def settle():
    import torch
    global _settled_at
    torch.cuda.synchronize()
    st = torch.cuda.memory_stats()
    mark = (st.get("segment.all.allocated", 0), st.get("segment.all.freed", 0))
    if mark != _settled_at:
        time.sleep(SETTLE_S)
        _settled_at = mark


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=64, help="requests (e4m3 headline point)")
    ap.add_argument("--splits", type=int, default=0, help="split-K count (0: library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the bf16 twin, the check overhead and the long-context point")
    ap.add_argument("--only", default=None,
                    help="comma-separated extras to run alone, without the headline point "
                         "(for profiling one workload): " + ", ".join(EXTRAS))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-from", default=COUNTERS_SUMMARY,
                    help="counter summary of the headline kernel (read for roofline.traffic)")
    ap.add_argument("--summarize-counters", default=None, metavar="PRESET",
                    help="turn the rocprofv3 --pmc runs of one counter preset into its summary "
                         "under profiles/ and exit: " + ", ".join(COUNTER_PRESETS))
    ap.add_argument("--pmc-dir", default=os.path.join("gpurun_out", "pmc"),
                    help="where the --pmc runs of --summarize-counters are")
    ap.add_argument("--summarize-kernel-stats", default=None, metavar="NAME",
                    help="turn a rocprofv3 --kernel-trace --stats run (--stats-dir) into "
                         "profiles/NAME_kernel_stats.md and exit: " + ", ".join(STATS_PRESETS))
    ap.add_argument("--stats-dir", default=os.path.join("gpurun_out", "prof"),
                    help="where the --kernel-trace --stats run of --summarize-kernel-stats is")
    return ap.parse_args()


def algorithmic_bytes(lens, Hq, Hkv, D, P, kv_elem_bytes, checked=True):
    """Bytes one attention launch must move: K+V of every attended token,
    the page-table entries, Q, out + lse, scales, lengths, status."""
    kv = sum(int(L) for L in lens) * Hkv * D * 2 * kv_elem_bytes
    table = sum((int(L) + P - 1) // P for L in lens) * 4
    B = len(lens)
    return (kv + table + B * Hq * D * 2 + B * Hq * (D + 1) * 4 + 2 * Hkv * 4 + B * 4
            + (B * 4 if checked else 0))


class Point:
    """One decode step's device state for a batch size and pool type."""

    def __init__(self, batch, kv_dtype, device, seed=SEED, workload=None):
        from paged_attention_fp8_amd import harness as H
        from paged_attention_fp8_amd import inputs as I
        from paged_attention_fp8_amd import ops
        self.ops, self.H = ops, H
        self.kv_dtype = kv_dtype
        elem = 1 if kv_dtype == ops.KV_FP8_E4M3 else 2
        self.w = workload if workload is not None else I.sweep_workload(batch, elem)
        log(f"drawing {self.w.name} ({'e4m3' if kv_dtype == ops.KV_FP8_E4M3 else 'bf16'})")
        self.inp = I.make_device_decode_inputs(self.w, seed, device)
        self.step = H.build_step(self.inp, kv_dtype, device, poison=False)
        log(f"cache built: {self.step.cache.num_pages} pages")
        self.sm = 1.0 / math.sqrt(self.w.head_dim)
        B, Hq, D = batch, self.w.q_heads, self.w.head_dim
        self.lens = self.inp.batch.context_lens
        # requests the tag check aborts read no pages: their K/V is not moved
        live = [0 if b in self.inp.stale else int(L) for b, L in enumerate(self.lens)]
        self.bytes = algorithmic_bytes(live, Hq, self.w.kv_heads, D, self.w.page_size, elem)

    def run(self, steps, warmup, splits, check=True, events=True, flush=False, fused=False,
            append_in_attention=False, prepared=False):
        """Time `steps` decode steps.  flush: before every step, read
        FLUSH_BYTES of other device memory so that no step finds the previous
        one's KV bytes in the last-level caches (the 256 MB MALL holds a
        whole batch of up to 8 requests); step times then come from HIP
        events around each step instead of the wall clock.  prepared (with
        append_in_attention): the check and the attention go through
        PreparedCalls, marshalled once before the loop."""
        import torch
        ops, H, st = self.ops, self.H, self.step
        B, Hq, D = st.batch.batch, self.w.q_heads, self.w.head_dim
        dev = st.q.device
        if splits == ops.BALANCED:
            S = -ops.default_balanced_groups(self.w.kv_heads)
        else:
            S = splits or ops.default_num_splits(B, self.w.kv_heads, st.batch.max_pages,
                                                 self.w.page_size)
            S = min(S, st.batch.max_pages)
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        status = torch.empty((B,), dtype=torch.int32, device=dev)
        nws = ops.workspace_bytes(B, Hq, D, S)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        junk = (torch.zeros(FLUSH_BYTES // 8, dtype=torch.int64, device=dev) if flush else None)
        if prepared:
            if not append_in_attention:
                raise ValueError("prepared runs take the append inside the attention launch")
            stream = torch.cuda.current_stream(dev).cuda_stream
            chk = (ops.prepare_page_tag_check(st.batch, self.w.page_size, st.page_tags,
                                              st.expected_tags, status) if check else None)
            att = ops.prepare_paged_decode_attn(st.cache, st.batch.with_status(status if check else None),
                                                st.q, self.sm, S, ws, out, lse, k_new=st.k_new,
                                                v_new=st.v_new)
        settle()

        def one(i=None):
            if junk is not None:
                junk.max()  # reads only: leaves no dirty lines to write back
            if i is not None and flush:
                sev[i][0].record()
            stat = None
            if prepared:
                if chk is not None:
                    chk.run(stream)
                if i is not None and events:
                    ev[i][0].record()
                att.run(stream)
                if i is not None and events:
                    ev[i][1].record()
                if i is not None and flush:
                    sev[i][1].record()
                return
            if append_in_attention:   # the append inside the attention launch
                if check:
                    stat = ops.page_tag_check(st.batch, self.w.page_size, st.page_tags,
                                              st.expected_tags, out=status)
                b = st.batch.with_status(stat)
                if i is not None and events:
                    ev[i][0].record()
                ops.paged_decode_attn(st.cache, b, st.q, self.sm, S, ws, out, lse,
                                      k_new=st.k_new, v_new=st.v_new)
                if i is not None and events:
                    ev[i][1].record()
                if i is not None and flush:
                    sev[i][1].record()
                return
            if fused:   # check and append in one launch
                stat = ops.kv_quant_append_checked(st.cache, st.batch, st.page_tags,
                                                   st.expected_tags, st.k_new, st.v_new, out=status)
                b = st.batch.with_status(stat)
            else:
                if check:
                    stat = ops.page_tag_check(st.batch, self.w.page_size, st.page_tags,
                                              st.expected_tags, out=status)
                b = st.batch.with_status(stat)
                ops.kv_quant_append(st.cache, b, st.k_new, st.v_new)
            if i is not None and events:
                ev[i][0].record()
            ops.paged_decode_attn(st.cache, b, st.q, self.sm, S, ws, out, lse)
            if i is not None and events:
                ev[i][1].record()
            if i is not None and flush:
                sev[i][1].record()

        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            one(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        attn_ms = [a.elapsed_time(b) for a, b in ev] if events else []
        ms = (statistics.mean(a.elapsed_time(b) for a, b in sev) if flush
              else 1e3 * wall / steps)
        return {"splits": S, "wall_s": wall, "ms_per_step": ms,
                "attn_ms": attn_ms, "out": out, "lse": lse, "status": status}


def cpu_baseline(point, target_s):
    """Time the CPU oracle on the first n requests of the same batch (n grows
    until one call takes about target_s seconds)."""
    import numpy as np
    import torch

    import oracle
    inp, w = point.inp, point.w
    Hkv, D, P = w.kv_heads, w.head_dim, w.page_size
    pool = oracle.Pool(oracle.KV_FP8, inp.num_pages, Hkv, P, D)
    table = inp.batch.page_table
    lens = inp.batch.context_lens
    q = inp.q.view(torch.int16).cpu().numpy().view(np.uint16)
    done = 0

    def ensure(n):
        nonlocal done
        for b in range(done, n):
            L = int(lens[b])
            k = inp.k_tokens[b, :L].view(torch.int16).cpu().numpy().view(np.uint16)
            v = inp.v_tokens[b, :L].view(torch.int16).cpu().numpy().view(np.uint16)
            oracle.kv_write(pool, table[b:b + 1], np.zeros(1, np.int32),
                            np.array([L], np.int32), k[None], v[None], inp.k_scale, inp.v_scale)
        done = max(done, n)

    def timed(n):
        ensure(n)
        log(f"cpu baseline: oracle on {n} request(s)")
        t0 = time.perf_counter()
        oracle.paged_attention(pool, q[:n], table[:n], lens[:n], point.sm, inp.k_scale,
                               inp.v_scale)
        return time.perf_counter() - t0

    n = 1
    t = timed(n)
    while t < 0.5 * target_s and n < len(lens):
        n = min(len(lens), max(n + 1, int(n * target_s / max(t, 1e-3))))
        t = timed(n)
    return {"value": n / t, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {n} of {len(lens)} requests of the same batch (all 64 heads, "
                      f"16384 tokens each), fp64 oracle, one call, {t:.1f} s"}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None where it is not given."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def long_context(args, dev):
    """4 requests of 262,144 tokens in 64 splits: the tag check's overhead on
    the clean batch (against the no-op tracker), and the batch with one
    stale request, which the check must abort while the others run."""
    import torch
    from paged_attention_fp8_amd import inputs as I
    from paged_attention_fp8_amd import ops
    w = I.WORKLOADS["gqa8_256k_b4"]
    pc = Point(w.batch, ops.KV_FP8_E4M3, dev, workload=I.scaled(w, stale_requests=0))
    rc = pc.run(args.steps, args.warmup, w.num_splits, check=True, flush=True)
    rn = pc.run(args.steps, args.warmup, w.num_splits, check=False, flush=True)
    clean_ms = statistics.mean(rc["attn_ms"])
    rd = pc.run(args.steps, args.warmup, 0, check=True, flush=True)
    dms = statistics.mean(rd["attn_ms"])
    res = {
        "workload": "gqa8_256k_b4: 4 requests x 262144 tokens, 64 query / 8 KV heads, head_dim 128, "
                    "64-token pages, 64 splits",
        "ms_per_step_checked": rc["ms_per_step"],
        "ms_per_step_no_tracker": rn["ms_per_step"],
        "check_overhead_pct": 100.0 * (rc["ms_per_step"] - rn["ms_per_step"]) / rn["ms_per_step"],
        # the check's cost per step in absolute terms: one check per decode
        # step shared by N layers costs this / N per layer call
        "check_us_per_step": 1e3 * (rc["ms_per_step"] - rn["ms_per_step"]),
        "attn_us": 1e3 * clean_ms,
        "attn_GBps": pc.bytes / (clean_ms * 1e-3) / 1e9,
        "attn_frac": pc.bytes / (clean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "default_splits": rd["splits"],
        "default_splits_attn_us": 1e3 * dms,
        "default_splits_attn_frac": pc.bytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    res.update(read_ceiling(dev, pc.bytes, args.steps))
    res["attn_over_read"] = res["attn_us"] / res["read_us"]
    del pc, rc, rn, rd
    torch.cuda.empty_cache()
    ps = Point(w.batch, ops.KV_FP8_E4M3, dev, workload=w)
    rs = ps.run(args.steps, args.warmup, w.num_splits, check=True, flush=True)
    flagged = [int(b) for b in torch.nonzero(rs["status"]).flatten().tolist()]
    if flagged != sorted(ps.inp.stale):
        raise SystemExit(f"long context: tag check flagged {flagged}, stale {ps.inp.stale}")
    ms = statistics.mean(rs["attn_ms"])
    res["stale_requests"] = flagged
    res["stale_ms_per_step"] = rs["ms_per_step"]
    res["stale_attn_GBps_live"] = ps.bytes / (ms * 1e-3) / 1e9
    del ps, rs
    torch.cuda.empty_cache()
    return res


def handoff(args, dev):
    """The prefill-to-decode hand-off: kv_quant_fill of 8 prompts of 8,192
    bf16 tokens (8 KV heads, head_dim 128) into e4m3 pages.  Per element it
    must read 2 bytes and write 1, for K and for V."""
    import torch
    from paged_attention_fp8_amd import harness as H
    from paged_attention_fp8_amd import inputs as I
    from paged_attention_fp8_amd import ops
    w = I.Workload("handoff_8k_b8", 8, 64, 8, 128, 64, 8192, 8192, pool_factor=1.0)
    inp = I.make_device_decode_inputs(w, SEED, dev)
    cache = H.new_cache(w, inp.num_pages, ops.KV_FP8_E4M3, dev, inp.k_scale, inp.v_scale, poison=False)
    batch, _, _ = H.upload_batch(inp.batch, inp.pool, dev)
    B, T = w.batch, w.max_len
    start = torch.zeros(B, dtype=torch.int32, device=dev)
    count = torch.full((B,), T, dtype=torch.int32, device=dev)
    k, v = inp.k_tokens[:, :T].contiguous(), inp.v_tokens[:, :T].contiguous()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    settle()
    for _ in range(args.warmup):
        ops.kv_quant_fill(cache, batch, start, count, k, v)
    for a, b in ev:
        a.record()
        ops.kv_quant_fill(cache, batch, start, count, k, v)
        b.record()
    torch.cuda.synchronize()
    ms = statistics.mean(a.elapsed_time(b) for a, b in ev)
    elems = B * T * w.kv_heads * w.head_dim
    nbytes = 2 * elems * (2 + 1) + B * (T // w.page_size) * 4 + 2 * B * 4 + 2 * w.kv_heads * 4
    del cache, inp, k, v
    torch.cuda.empty_cache()
    res = {"workload": "8 prompts x 8192 bf16 tokens, 8 KV heads, head_dim 128, 64-token pages -> e4m3",
           "kernel": "kv_fill_kernel<e4m3, 128>", "us": 1e3 * ms, "algorithmic_bytes": nbytes,
           "GBps": nbytes / (ms * 1e-3) / 1e9, "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    # the bare stream of the same shape: read the 2-byte source, write half
    res.update(_read_write_ceiling(_ceiling(dev), 2 * elems * 2, 2, args.steps, args.warmup))
    res["over_read_write"] = res["us"] / res["read_write_us"]
    return res


def decode_loop(args, dev):
    """Continuous decode under the 2 GiB pool budget: 128 requests of 16,384
    tokens in total (prompt handed over by kv_quant_fill, then 64-192 decode
    steps each), admitted first come first served while pages are free; each
    step is kv_quant_append_checked + attention over 64 slots.  Run once with
    an e4m3 pool and once with a bf16 pool of the same bytes."""
    import numpy as np
    import torch
    from paged_attention_fp8_amd import decode_loop as DL
    from paged_attention_fp8_amd import inputs as I
    from paged_attention_fp8_amd import ops
    g = np.random.default_rng(SEED + 7)
    dec = g.integers(64, 193, 128)
    gen = torch.Generator(device=dev)
    gen.manual_seed(SEED + 8)
    sample = torch.randn(1 << 22, generator=gen, device=dev).to(torch.bfloat16).float()
    scale = I.fp8_scale_from_amax(np.full(8, float(sample.abs().max()), np.float32))
    res = {}
    for kv_dtype, name in ((ops.KV_FP8_E4M3, "e4m3"), (ops.KV_BF16, "bf16")):
        loop = DL.DecodeLoop(kv_dtype, I.SWEEP_BUDGET_BYTES, 64, 8, 128, 64, 64, 16384, dev,
                             SEED, scale, scale)
        for rid, d in enumerate(dec):
            loop.submit(DL.Request(rid, 16384 - int(d), int(d)))
        settle()
        stats = []
        t0 = time.perf_counter()
        while (loop.queue or any(r is not None for r in loop.slots)) and len(stats) < 4000:
            stats.append(loop.step())
        wall = time.perf_counter() - t0
        tokens = sum(st.active for st in stats)
        gpu_s = sum(st.gpu_ms for st in stats) * 1e-3
        res[name] = {
            "pool_pages": loop.num_pages,
            "max_concurrent": loop.max_active,
            "waiting_after_first_step": stats[0].waiting,
            "steps": len(stats),
            "finished": sum(1 for r in loop.finished if not r.terminated),
            "terminated": sum(1 for r in loop.finished if r.terminated),
            "decode_tokens": tokens,
            "decode_tokens_per_gpu_s": tokens / gpu_s,
            "mean_step_gpu_ms": 1e3 * gpu_s / len(stats),
            "wall_s": wall,
        }
        del loop
        torch.cuda.empty_cache()
    return {"workload": "128 requests x 16384 tokens (prompt + 64..192 decode steps), GQA 64/8, "
                        "head_dim 128, 64-token pages, 2 GiB pool, 64 slots", **res}


def int4_decode(args, dev):
    """Decode-time weight streaming with INT4 weights: y = x . W^T for 8
    distinct 28672 x 8192 weight matrices in turn (940 MB of int4 weights, far
    beyond the MALL), at 1, 8, 16, 32 and 64 rows of x (concurrent requests)."""
    import torch
    from paged_attention_fp8_amd import ops
    N, K, layers = 28672, 8192, 8
    gen = torch.Generator(device=dev)
    gen.manual_seed(SEED + 11)
    ws = [torch.randint(0, 256, (N * K // 2,), generator=gen, device=dev, dtype=torch.uint8)
          for _ in range(layers)]
    ss = [(torch.rand((K // 128, N), generator=gen, device=dev) * 0.05 + 1e-3).to(torch.bfloat16)
          for _ in range(layers)]
    res = []
    for M in (1, 8, 16, 32, 64):
        x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        settle()
        for _ in range(args.warmup):
            for i in range(layers):
                ops.int4_gemv(x, ws[i], ss[i], N, K, out=y)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            for i in range(layers):
                ops.int4_gemv(x, ws[i], ss[i], N, K, out=y)
            b.record()
        torch.cuda.synchronize()
        ms = statistics.mean(a.elapsed_time(b) for a, b in ev) / layers
        nbytes = N * K // 2 + (K // 128) * N * 2 + M * K * 2 + M * N * 4
        res.append({"rows": M, "us_per_matrix": 1e3 * ms,
                    "GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                    "TFLOPs": 2.0 * M * N * K / (ms * 1e-3) / 1e12})
    del ws, ss
    torch.cuda.empty_cache()
    # the bare read of one matrix's weights and scales, 8 disjoint copies
    # back to back, timed like the GEMVs
    wbytes = N * K // 2 + (K // 128) * N * 2
    ceil = _ceiling(dev).back_to_back(wbytes, layers, args.steps)
    for r in res:
        r["over_read"] = r["us_per_matrix"] / ceil["read_us"]
    return {"workload": "8 int4 weight matrices 28672 x 8192 (bf16 scale per 128 inputs), "
                        "bf16 activations, fp32 output", "read_ceiling": ceil,
            "kernel": "int4_gemv_row_kernel (1 row), int4_gemv_kernel (2-16 rows), "
                      "int4_gemv_wide_kernel (17-64 rows)", "points": res}


def fp8_vs_bf16(args, dev):
    """The ragged workload (32 requests of 1k-32k tokens, GQA 64/8, 64-token
    pages, fragmented pool) on an e4m3 cache and on a bf16 cache built from
    the identical bf16 source: attention time of each, with the library's
    default splits and with the balanced partition (negative `splits`: W
    work-groups per KV head sharing all requests' pages equally), and how far
    the e4m3 outputs lie from the bf16 ones (a statistic, not a gate: the
    pages call the two indistinguishable in accuracy without a kernel-level
    figure)."""
    import torch
    from paged_attention_fp8_amd import inputs as I
    from paged_attention_fp8_amd import ops
    w = I.WORKLOADS["gqa8_ragged_32k"]
    runs = {}
    for kv_dtype, name in ((ops.KV_FP8_E4M3, "e4m3"), (ops.KV_BF16, "bf16")):
        pt = Point(w.batch, kv_dtype, dev, workload=w)
        for mode in (0, ops.BALANCED):
            r = pt.run(args.steps, args.warmup, mode, flush=True)
            ms = statistics.mean(r["attn_ms"])
            res = {"attn_us": 1e3 * ms, "attn_GBps": pt.bytes / (ms * 1e-3) / 1e9,
                   "attn_frac": pt.bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "splits": r["splits"]}
            _with_ceiling(res, dev, pt.bytes, args.steps)
            if mode == 0:
                runs[name] = dict(res, out=r["out"].clone(), lse=r["lse"].clone())
            else:
                runs[name]["balanced"] = res
            del r
        del pt
        torch.cuda.empty_cache()
    d = (runs["e4m3"]["out"] - runs["bf16"]["out"]).abs()
    ref = runs["bf16"]["out"].abs()
    dl = (runs["e4m3"]["lse"] - runs["bf16"]["lse"]).abs()
    res = {"workload": "gqa8_ragged_32k: 32 requests x U[1024, 32768] tokens, 64 query / 8 KV heads, "
                       "head_dim 128, 64-token pages, fragmented pool, identical bf16 source"}
    for name in ("e4m3", "bf16"):
        res[name] = {k: v for k, v in runs[name].items() if k not in ("out", "lse")}
    res["out_abs_diff"] = {"max": float(d.max()), "mean": float(d.mean()),
                           "p99": float(torch.quantile(d.flatten()[:1 << 24].float(), 0.99))}
    res["out_rel_diff_mean"] = float((d.sum() / ref.sum()))
    res["lse_abs_diff_max"] = float(dl.max())
    return res


def _attn_point(pt, rr):
    """Figures of one timed point: attention launch (HIP events, flushed
    caches), the step around it, and the share of peak HBM bandwidth."""
    ms = statistics.mean(rr["attn_ms"])
    B = pt.step.batch.batch
    return {"attn_us": 1e3 * ms, "attn_us_median": 1e3 * statistics.median(rr["attn_ms"]),
            "attn_GBps": pt.bytes / (ms * 1e-3) / 1e9,
            "attn_frac": pt.bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "ms_per_step": rr["ms_per_step"], "tokens_per_s": B / (rr["ms_per_step"] * 1e-3),
            "splits": rr["splits"], "algorithmic_bytes": pt.bytes}


class ReadCeiling:
    """What the memory system delivers for a point's byte count: the
    library's bare non-temporal read (ops.stream_read) of the same number of
    bytes, each launch after the same 1 GiB flush and timed with the same HIP
    events as the attention; the best of a few work-group counts is kept.
    No kernel that must read those bytes once can beat it under this timing,
    so attn_us / read_us says how much of the attention's time is more than
    the read itself."""
    CAPACITY = 5 << 29          # 2.5 GiB; the largest point reads 2.15 GB
    GRIDS = (256, 512, 1024)

    def __init__(self, dev):
        import torch
        from paged_attention_fp8_amd import ops
        self.ops = ops
        self.buf = torch.full((self.CAPACITY,), 0x5A, dtype=torch.uint8, device=dev)
        self.junk = torch.zeros(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
        self.sink = torch.empty(max(self.GRIDS) * ops.STREAM_READ_THREADS, dtype=torch.int32,
                                device=dev)
        self.done = {}

    def __call__(self, nbytes, steps):
        import torch
        n = min(nbytes, self.CAPACITY) // self.ops.STREAM_READ_TILE * self.ops.STREAM_READ_TILE
        if n not in self.done:
            view = self.buf[:n]
            best = None
            for g in self.GRIDS:
                self.ops.stream_read(view, g, self.sink)
                settle()
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(steps)]
                for a, b in ev:
                    self.junk.max()
                    a.record()
                    self.ops.stream_read(view, g, self.sink)
                    b.record()
                torch.cuda.synchronize()
                us = 1e3 * statistics.mean(a.elapsed_time(b) for a, b in ev)
                if best is None or us < best[0]:
                    best = (us, g)
            self.done[n] = {"read_us": best[0], "read_work_groups": best[1], "read_bytes": n,
                            "read_frac": n / (best[0] * 1e-6) / 1e9 / PEAK_HBM_GBS}
        return dict(self.done[n])

    def back_to_back(self, nbytes, count, steps):
        """count bare reads of nbytes each over disjoint slices of the
        buffer, launched back to back and timed together (no flush: the
        slices together exceed the MALL), per-launch mean; best grid."""
        import torch
        t = self.ops.STREAM_READ_TILE
        n = nbytes // t * t
        if n * count > self.CAPACITY:
            raise ValueError("back_to_back: %d x %d bytes exceed the buffer" % (count, n))
        views = [self.buf[i * n:(i + 1) * n] for i in range(count)]
        best = None
        for g in self.GRIDS:
            for v in views:
                self.ops.stream_read(v, g, self.sink)
            settle()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                a.record()
                for v in views:
                    self.ops.stream_read(v, g, self.sink)
                b.record()
            torch.cuda.synchronize()
            us = 1e3 * statistics.mean(a.elapsed_time(b) for a, b in ev) / count
            if best is None or us < best[0]:
                best = (us, g)
        return {"read_us": best[0], "read_work_groups": best[1], "read_bytes": n,
                "read_frac": n / (best[0] * 1e-6) / 1e9 / PEAK_HBM_GBS}


# A stream that also writes runs fastest on fine grids (one 16 KiB tile per
# work-group at the hand-off's size: 57.7 us against 62.1 us at 1024), so its
# ceiling tries them too; the read-only stream is best at 256-512.
READ_WRITE_GRIDS = (256, 1024, 4096, 16384)


def _read_write_ceiling(rc, src_bytes, ratio, steps, warmup):
    """The bare read of src_bytes with a write of src_bytes / ratio
    (ops.stream_read_write), launched and timed like the hand-off: back to
    back, HIP events per launch, no flush; best grid."""
    import torch
    t = rc.ops.STREAM_READ_TILE
    n = src_bytes // t * t
    src, dst = rc.buf[:n], rc.buf[rc.CAPACITY - n // ratio:]
    if n + n // ratio > rc.CAPACITY:
        raise ValueError("read_write: %d bytes exceed the buffer" % n)
    best = None
    for g in READ_WRITE_GRIDS:
        rc.ops.stream_read_write(src, dst, g)
        settle()
        for _ in range(warmup):
            rc.ops.stream_read_write(src, dst, g)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record()
            rc.ops.stream_read_write(src, dst, g)
            b.record()
        torch.cuda.synchronize()
        us = 1e3 * statistics.mean(a.elapsed_time(b) for a, b in ev)
        if best is None or us < best[0]:
            best = (us, g)
    moved = n + n // ratio
    return {"read_write_us": best[0], "read_write_work_groups": best[1], "read_bytes": n,
            "write_bytes": n // ratio, "read_write_frac": moved / (best[0] * 1e-6) / 1e9 / PEAK_HBM_GBS}


_read_ceilings = {}


def _ceiling(dev):
    if dev not in _read_ceilings:
        _read_ceilings[dev] = ReadCeiling(dev)
    return _read_ceilings[dev]


def read_ceiling(dev, nbytes, steps):
    """ReadCeiling figures for nbytes, with attn_us to be set beside them."""
    return _ceiling(dev)(nbytes, steps)


def _with_ceiling(entry, dev, nbytes, steps):
    entry.update(read_ceiling(dev, nbytes, steps))
    entry["attn_over_read"] = entry["attn_us"] / entry["read_us"]
    return entry


def concurrency_sweep(args, dev, head=None):
    """The concurrency table of the pages' KV-cache section: 1, 8, 16, 32 and
    64 requests of 16,384 tokens (GQA 64/8, head_dim 128, 64-token pages) in
    the 2 GiB pool, e4m3 and bf16, library-default splits.  bf16 at 64
    requests does not fit the pool: the allocator refuses it.  Every step is
    preceded by a 1 GiB read of other memory, so that no point runs from the
    256 MB MALL; step = check + append + attention."""
    import torch
    from paged_attention_fp8_amd import inputs as I
    from paged_attention_fp8_amd import ops
    points = []
    for kv_dtype, name in ((ops.KV_FP8_E4M3, "e4m3"), (ops.KV_BF16, "bf16")):
        for b in (1, 8, 16, 32, 64):
            entry = {"dtype": name, "batch": b}
            if head is not None and kv_dtype == head.kv_dtype and b == head.step.batch.batch:
                pt = head
            else:
                try:
                    pt = Point(b, kv_dtype, dev)
                except I.PoolExhausted as e:
                    entry["result"] = f"out of pool memory ({e})"
                    points.append(entry)
                    continue
            entry.update(_attn_point(pt, pt.run(args.steps, args.warmup, 0, flush=True)))
            _with_ceiling(entry, dev, pt.bytes, args.steps)
            points.append(entry)
            log(f"sweep {name} B={b}: {entry['attn_us']:.1f} us, {100 * entry['attn_frac']:.1f}%; "
                f"bare read {entry['read_us']:.1f} us, {100 * entry['read_frac']:.1f}%")
            if pt is not head:
                del pt
                torch.cuda.empty_cache()
    return {"workload": "gqa8_16k_b{1,8,16,32,64}: B requests x 16384 tokens, 64 query / 8 KV heads, "
                        "head_dim 128, 64-token pages, 2 GiB pool, flushed caches", "points": points}


def gqa4_4k(args, dev):
    """8 requests of 4,096 tokens, GQA 32/8, head_dim 128, 16-token pages,
    1% of K/V elements x20 (saturating the e4m3 range): the small-page,
    latency-bound workload; library-default splits, flushed caches."""
    import torch
    from paged_attention_fp8_amd import inputs as I
    from paged_attention_fp8_amd import ops
    w = I.WORKLOADS["gqa4_4k_outliers"]
    res = {"workload": "gqa4_4k_outliers: 8 requests x 4096 tokens, 32 query / 8 KV heads, head_dim 128, "
                       "16-token pages, 1% outliers x20, flushed caches"}
    for kv_dtype, name in ((ops.KV_FP8_E4M3, "e4m3"), (ops.KV_BF16, "bf16")):
        pt = Point(w.batch, kv_dtype, dev, workload=w)
        res[name] = _attn_point(pt, pt.run(args.steps, args.warmup, 0, flush=True))
        _with_ceiling(res[name], dev, pt.bytes, args.steps)
        log(f"gqa4_4k {name}: {res[name]['attn_us']:.1f} us, {100 * res[name]['attn_frac']:.1f}%; "
            f"bare read {res[name]['read_us']:.1f} us, {100 * res[name]['read_frac']:.1f}%")
        del pt
        torch.cuda.empty_cache()
    return res


def _mha_g1_workload():
    from paged_attention_fp8_amd import inputs as I
    return I.Workload("mha_g1_16k_b8", 8, 32, 32, 128, 64, 16384, 16384, pool_factor=1.0)


def mha_g1(args, dev):
    """One query head per KV head (one live MFMA column of the group): 8
    requests of 16,384 tokens, 32 heads, head_dim 128, 64-token pages,
    e4m3 and bf16, library-default splits, flushed caches, each beside the
    bare read of its bytes."""
    import torch
    from paged_attention_fp8_amd import inputs as I
    from paged_attention_fp8_amd import ops
    w = _mha_g1_workload()
    res = {"workload": "mha_g1_16k_b8: 8 requests x 16384 tokens, 32 query heads = 32 KV heads, head_dim 128, "
                       "64-token pages, flushed caches"}
    for kv_dtype, name in ((ops.KV_FP8_E4M3, "e4m3"), (ops.KV_BF16, "bf16")):
        pt = Point(w.batch, kv_dtype, dev, workload=w)
        res[name] = _attn_point(pt, pt.run(args.steps, args.warmup, 0, flush=True))
        _with_ceiling(res[name], dev, pt.bytes, args.steps)
        log(f"mha_g1 {name}: {res[name]['attn_us']:.1f} us, {100 * res[name]['attn_frac']:.1f}%; "
            f"bare read {res[name]['read_us']:.1f} us, {100 * res[name]['read_frac']:.1f}%")
        del pt
        torch.cuda.empty_cache()
    return res


def _pmc_values(directory, counter, kernel_substr):
    """Per-dispatch values of one counter for kernels whose name contains
    kernel_substr, from a rocprofv3 --pmc csv run directory."""
    import csv
    vals = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter and kernel_substr in row.get("Kernel_Name", ""):
                    vals.append(float(row["Counter_Value"]))
    return vals


# Counter presets: one per kernel the bench reports.  Each names the bench
# arguments that run the kernel's workload, the kernel (a substring of its
# full name), the sources it is built from, and its algorithmic bytes per
# launch, computed on the host from the seeded workload definition.
def _attn_workload_bytes(w, seed, kv_elem_bytes, checked=True):
    from paged_attention_fp8_amd import inputs as I
    lens = I.context_lengths(w, seed)
    stale = set(I.stale_requests(w, seed, len(lens)))
    live = [0 if b in stale else int(L) for b, L in enumerate(lens)]
    return algorithmic_bytes(live, w.q_heads, w.kv_heads, w.head_dim, w.page_size, kv_elem_bytes,
                             checked)


def _int4_bytes(M, N=28672, K=8192):
    return N * K // 2 + (K // 128) * N * 2 + M * K * 2 + M * N * 4


def _handoff_bytes(B=8, T=8192, Hkv=8, D=128, P=64):
    elems = B * T * Hkv * D
    return 2 * elems * (2 + 1) + B * (T // P) * 4 + 2 * B * 4 + 2 * Hkv * 4


def _preset_bytes(name):
    from paged_attention_fp8_amd import inputs as I
    if name == "decode_attn_e4m3_gqa8_16k_b64":
        return _attn_workload_bytes(I.sweep_workload(64, 1), SEED, 1)
    if name == "decode_attn_wave_e4m3_gqa8_256k_b4_s64":
        return _attn_workload_bytes(I.scaled(I.WORKLOADS["gqa8_256k_b4"], stale_requests=0), SEED, 1)
    if name == "splitk_combine_gqa8_256k_b4_s64":
        B, Hq, S, D = 4, 64, 64, 128
        return B * Hq * S * (D + 1) * 4 + B * Hq * (D + 1) * 4 + B * 4
    if name == "decode_attn_small_pages_e4m3_gqa4_4k":
        return _attn_workload_bytes(I.WORKLOADS["gqa4_4k_outliers"], SEED, 1)
    if name == "decode_attn_bal_e4m3_ragged_32k":
        return _attn_workload_bytes(I.WORKLOADS["gqa8_ragged_32k"], SEED, 1)
    if name == "decode_attn_e4m3_mha_16k_b8":
        return _attn_workload_bytes(_mha_g1_workload(), SEED, 1)
    if name == "kv_fill_e4m3_handoff_8k_b8":
        return _handoff_bytes()
    if name == "int4_gemv_row_28672x8192_m1":
        return _int4_bytes(1)
    if name == "int4_gemv_28672x8192_m64":
        return _int4_bytes(64)
    if name == "int4_gemv_28672x8192_m16":
        return _int4_bytes(16)
    raise KeyError(name)


_ATTN = ("decode_attn.hip", "pafp8_device.hpp", "attn_params.hpp")
COUNTER_PRESETS = {
    "decode_attn_e4m3_gqa8_16k_b64": dict(
        what="e4m3 paged decode attention, 64 requests x 16384 tokens (the headline launch)",
        args="--steps 5 --warmup 2 --no-cpu-baseline --no-extras",
        kernel="decode_attn_mfma_kernel<false, 128, true, false, true>", sources=_ATTN),
    "decode_attn_wave_e4m3_gqa8_256k_b4_s64": dict(
        what="e4m3 attention in wave-per-split mode, 4 requests x 262144 tokens, 64 splits "
             "(median launch: the clean batch; the stale-request batch reads 3/4 of it)",
        args="--only long_context --steps 3 --warmup 1",
        kernel="decode_attn_mfma_wave_kernel<false, 128, true, true>", sources=_ATTN),
    "splitk_combine_gqa8_256k_b4_s64": dict(
        what="split-K combine of 64 splits, 4 requests x 64 query heads x 128 dims",
        args="--only long_context --steps 3 --warmup 1",
        kernel="splitk_combine_wg_kernel<128>", sources=("splitk_combine.hip", "pafp8_device.hpp")),
    "decode_attn_small_pages_e4m3_gqa4_4k": dict(
        what="e4m3 attention over 16-token pages, 8 requests x 4096 tokens, GQA 32/8, 4 splits",
        args="--only gqa4_4k --steps 3 --warmup 1",
        kernel="decode_attn_mfma_kernel<false, 128, false, false, true>", sources=_ATTN),
    "decode_attn_bal_e4m3_ragged_32k": dict(
        what="e4m3 attention, balanced partition, 32 ragged requests of 1k-32k tokens",
        args="--only fp8_vs_bf16 --steps 3 --warmup 1",
        kernel="decode_attn_bal_mfma_kernel<false, 128, true, false, true>", sources=_ATTN),
    "decode_attn_e4m3_mha_16k_b8": dict(
        what="e4m3 attention with one query head per KV head, 8 requests x 16384 tokens, 32 heads",
        args="--only mha_g1 --steps 3 --warmup 1",
        kernel="decode_attn_mfma_kernel<false, 128, true, false, true>", sources=_ATTN),
    "kv_fill_e4m3_handoff_8k_b8": dict(
        what="kv_quant_fill of 8 prompts x 8192 bf16 tokens into e4m3 pages",
        args="--only prefill_handoff --steps 3 --warmup 1",
        kernel="kv_fill_kernel<false, 128>",
        sources=("kv_write.hip", "pafp8_quant.hpp", "pafp8_append.hpp", "pafp8_device.hpp")),
    "int4_gemv_row_28672x8192_m1": dict(
        what="INT4 weight-streaming GEMV, one row of x, 28672 x 8192 weights",
        args="--only int4_decode_gemv --steps 3 --warmup 1",
        kernel="int4_gemv_row_kernel", sources=("int4_gemv.hip", "pafp8_device.hpp")),
    "int4_gemv_28672x8192_m16": dict(
        what="INT4 weight-streaming GEMV, 8 and 16 rows of x (bytes counted at 16), 28672 x 8192 weights",
        args="--only int4_decode_gemv --steps 3 --warmup 1",
        kernel="int4_gemv_kernel<1, 8, true, 8>", sources=("int4_gemv.hip", "pafp8_device.hpp")),
    "int4_gemv_28672x8192_m64": dict(
        what="INT4 weight-streaming GEMV, 64 rows of x, 28672 x 8192 weights",
        args="--only int4_decode_gemv --steps 3 --warmup 1",
        kernel="int4_gemv_wide_kernel<2>", sources=("int4_gemv.hip", "pafp8_device.hpp")),
}


def preset_hash(sources) -> str:
    """Hash of a kernel's sources: counter figures taken on other sources are stale."""
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "paged_attention_fp8_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_summary_path(preset):
    return os.path.join(ROOT, "profiles", f"{preset}_counters.md")


def summarize_counters(preset, pmc_dir, out_path=None):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of one preset's kernel, each
    scaled by what the same counter reads for a plain 1 GiB device copy, with
    the kernel's algorithmic bytes beside them."""
    cfg = COUNTER_PRESETS[preset]
    d = lambda tag: os.path.join(pmc_dir, tag)
    f = _pmc_values(d(f"{preset}_fetch"), "FETCH_SIZE", cfg["kernel"])
    w = _pmc_values(d(f"{preset}_write"), "WRITE_SIZE", cfg["kernel"])
    cf = _pmc_values(d("copy_fetch"), "FETCH_SIZE", "copy")
    cw = _pmc_values(d("copy_write"), "WRITE_SIZE", "copy")
    if not (f and w and cf and cw):
        raise SystemExit(f"{preset}: missing counter rows: fetch {len(f)} write {len(w)} "
                         f"copy {len(cf)}/{len(cw)}")
    # the copy moves COPY_BYTES each way; its largest dispatches are the copies
    cf_kib, cw_kib = max(cf), max(cw)
    kf = COPY_BYTES / (cf_kib * 1024.0)
    kw = COPY_BYTES / (cw_kib * 1024.0)
    fetch = statistics.median(f) * 1024.0 * kf
    write = statistics.median(w) * 1024.0 * kw
    alg = _preset_bytes(preset)
    run = lambda c, tag, a: [f"    rocprofv3 --pmc {c} --output-format csv -d {d(tag)} -o run -- \\",
                             f"        python bench.py {a}"]
    lines = [f"# HBM traffic counters: {cfg['what']}", "",
             "Commands (MI355X, repository root; one counter per run):", ""]
    lines += run("FETCH_SIZE", f"{preset}_fetch", cfg["args"])
    lines += run("WRITE_SIZE", f"{preset}_write", cfg["args"])
    lines += run("FETCH_SIZE", "copy_fetch", "--copy-calibration")
    lines += run("WRITE_SIZE", "copy_write", "--copy-calibration")
    lines += [f"    python bench.py --summarize-counters {preset} --pmc-dir {pmc_dir}", "",
              f"kernel: {cfg['kernel']}",
              f"dispatches: {len(f)} (FETCH_SIZE), {len(w)} (WRITE_SIZE)",
              f"FETCH_SIZE median: {statistics.median(f):.1f} KiB per dispatch "
              f"(min {min(f):.1f}, max {max(f):.1f})",
              f"WRITE_SIZE median: {statistics.median(w):.1f} KiB per dispatch "
              f"(min {min(w):.1f}, max {max(w):.1f})",
              f"copy calibration: 1 GiB copy reads FETCH_SIZE {cf_kib:.1f} KiB, WRITE_SIZE {cw_kib:.1f} KiB",
              f"scale factors (known bytes / counter bytes): fetch {kf:.4f}, write {kw:.4f}",
              f"traffic_bytes_per_launch: {fetch + write:.0f}",
              f"fetch_bytes_per_launch: {fetch:.0f}",
              f"write_bytes_per_launch: {write:.0f}",
              f"algorithmic_bytes_per_launch: {alg}",
              f"traffic_over_algorithmic: {(fetch + write) / alg:.4f}",
              f"source_hash: {preset_hash(cfg['sources'])}", ""]
    out_path = out_path or counter_summary_path(preset)
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


# Kernel-trace summaries: the bench arguments profiled and what the summary is of.
STATS_PRESETS = {
    "decode_attn_e4m3_gqa8_16k_b64": dict(
        what="e4m3 paged decode attention, 64 requests x 16384 tokens (the headline step: "
             "page_tag_check + kv_quant_append + paged_decode_attn_fp8)",
        args="--steps 20 --warmup 5 --no-cpu-baseline --no-extras",
        headline="decode_attn_mfma_kernel<false, 128, true, false, true>"),
    "path_extras": dict(
        what="every kernel of the library under the full bench run (headline, bf16 twin, "
             "concurrency sweep, 4k small pages, long context, hand-off, decode loop, INT4, ragged)",
        args="--steps 20 --warmup 5 --no-cpu-baseline", headline=None),
}


def summarize_kernel_stats(name, stats_dir, out_path=None):
    """The library's kernels from a rocprofv3 --kernel-trace --stats run: calls
    and durations, and for the headline preset the attention launch's
    algorithmic bytes over its average duration."""
    import csv
    cfg = STATS_PRESETS[name]
    paths = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {stats_dir}")
    rows = []
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if "pafp8::" in r["Name"]:
                    rows.append(r)
    def short(n):   # "void pafp8::(anonymous namespace)::k<...>(args)" -> "k<...>"
        n = n.replace("pafp8::(anonymous namespace)::", "").replace("void ", "", 1)
        return n.split("(")[0]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel statistics: {cfg['what']}", "",
             "Command (MI355X, repository root):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d {stats_dir} -o run -- \\",
             f"        python bench.py {cfg['args']}",
             f"    python bench.py --summarize-kernel-stats {name} --stats-dir {stats_dir}", "",
             "Calls include warm-up and cache-building launches.", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} |")
    if cfg["headline"]:
        h = [r for r in rows if cfg["headline"] in r["Name"]]
        if h:
            avg = float(h[0]["AverageNs"])
            alg = _preset_bytes("decode_attn_e4m3_gqa8_16k_b64")
            lines += ["", f"headline kernel: {cfg['headline']}",
                      f"average_duration_ns: {avg:.0f}",
                      f"algorithmic_bytes_per_launch: {alg}",
                      f"achieved_GBps: {alg / avg:.1f}",
                      f"frac_of_8TBps: {alg / avg / PEAK_HBM_GBS:.4f}"]
    lines.append("")
    out_path = out_path or os.path.join(ROOT, "profiles", f"{name}_kernel_stats.md")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def read_traffic(summary_path):
    """HBM bytes per attention launch from the committed counter summary, or
    None when there is none or it was taken on other kernel sources."""
    if not summary_path or not os.path.exists(summary_path):
        return None
    vals = {}
    with open(summary_path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != preset_hash(_ATTN):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    n = COPY_BYTES
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


# the extras of the default run (and of --only), in run order
EXTRAS = {
    "concurrency_sweep": concurrency_sweep,
    "gqa4_4k": gqa4_4k,
    "mha_g1": mha_g1,
    "long_context": long_context,
    "prefill_handoff": handoff,
    "decode_loop": decode_loop,
    "int4_decode_gemv": int4_decode,
    "fp8_vs_bf16": fp8_vs_bf16,
}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); decode attention "
              "shards by request or KV head with no exchange between GPUs, so the one-GPU figure "
              "is the per-GPU throughput",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_kernel_stats:
        summarize_kernel_stats(args.summarize_kernel_stats, args.stats_dir)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.pmc_dir)
        return
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    from paged_attention_fp8_amd import ops
    dev = torch.device("cuda:0")
    if args.only:
        names = [n.strip() for n in args.only.split(",") if n.strip()]
        unknown = [n for n in names if n not in EXTRAS]
        if unknown:
            raise SystemExit(f"--only: unknown extras {unknown} (known: {', '.join(EXTRAS)})")
        print(json.dumps({n: EXTRAS[n](args, dev) for n in names}), flush=True)
        return

    p = Point(args.batch, ops.KV_FP8_E4M3, dev)
    r = p.run(args.steps, args.warmup, args.splits)
    log(f"e4m3 B={args.batch}: {r['ms_per_step']:.3f} ms/step")
    if not torch.all(r["status"] == 0):
        raise SystemExit("tag check flagged requests in a clean batch")
    if not torch.isfinite(r["out"]).all():
        raise SystemExit("non-finite attention output")
    attn_ms = statistics.mean(r["attn_ms"])
    achieved = p.bytes / (attn_ms * 1e-3) / 1e9
    B = args.batch
    result = {
        "metric": METRIC,
        "value": B / (r["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"gqa8_16k_b{B}: {B} requests x 16384 tokens, 64 query / 8 KV heads, "
                        "head_dim 128, 64-token pages, 2 GiB e4m3 pool, tag check + append + attention",
            "batch": B, "context": 16384, "q_heads": 64, "kv_heads": 8, "head_dim": 128,
            "page_size": 64, "num_splits": r["splits"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": read_traffic(args.traffic_from),
            "kernel": "decode_attn_mfma_kernel<e4m3, 128>",
            "algorithmic_bytes_per_launch": p.bytes,
            "launch_ms_mean": attn_ms,
            "launch_ms_median": statistics.median(r["attn_ms"]),
            "launch_ms_p10_p90": [sorted(r["attn_ms"])[len(r["attn_ms"]) // 10],
                                  sorted(r["attn_ms"])[(9 * len(r["attn_ms"])) // 10]],
        },
        "context_tokens_per_s": float(sum(int(L) for L in p.lens)) / (attn_ms * 1e-3),
    }
    if result["roofline"]["traffic"] is not None:
        # the counters' HBM bytes over the same mean launch time
        result["roofline"]["traffic_GBps"] = result["roofline"]["traffic"] / (attn_ms * 1e-3) / 1e9
    if not args.no_extras:
        r0 = p.run(args.steps, args.warmup, args.splits, check=False)
        result["check_overhead_pct"] = 100.0 * (r["ms_per_step"] - r0["ms_per_step"]) / r0["ms_per_step"]
        result["check_us_per_step"] = 1e3 * (r["ms_per_step"] - r0["ms_per_step"])
        result["no_tracker_ms_per_step"] = r0["ms_per_step"]
        rf = p.run(args.steps, args.warmup, args.splits, fused=True)
        if not torch.all(rf["status"] == 0):
            raise SystemExit("fused check flagged requests in a clean batch")
        result["fused_check"] = {
            "ms_per_step": rf["ms_per_step"],
            "check_overhead_pct": 100.0 * (rf["ms_per_step"] - r0["ms_per_step"]) / r0["ms_per_step"],
        }
        del r0, rf
        # the append inside the attention launch: same pool bytes and outputs,
        # one launch fewer (at 64 requests, and at one request where launches
        # weigh most)
        ra = p.run(args.steps, args.warmup, args.splits, append_in_attention=True)
        one = Point(1, ops.KV_FP8_E4M3, dev)
        r1s = one.run(args.steps, args.warmup, 0)
        r1f = one.run(args.steps, args.warmup, 0, append_in_attention=True)
        r1c = one.run(args.steps, args.warmup, 0, fused=True)
        r1p = one.run(args.steps, args.warmup, 0, append_in_attention=True, prepared=True, events=False)
        result["append_in_attention"] = {
            "step": "tag check + attention with the append in its launch, against tag check + "
                    "append + attention (and, at one request, the check inside the append launch)",
            "b64": {"ms_per_step": ra["ms_per_step"], "separate_ms_per_step": r["ms_per_step"],
                    "tokens_per_s": B / (ra["ms_per_step"] * 1e-3)},
            "b1": {"ms_per_step": r1f["ms_per_step"], "separate_ms_per_step": r1s["ms_per_step"],
                   "checked_append_ms_per_step": r1c["ms_per_step"],
                   # the same step through prepared calls (argument checks
                   # and marshalling done once; still eager launches)
                   "prepared_ms_per_step": r1p["ms_per_step"],
                   "tokens_per_s": 1 / (r1f["ms_per_step"] * 1e-3), "splits": r1f["splits"]},
        }
        del ra, one, r1s, r1f, r1c, r1p
        q = Point(32, ops.KV_BF16, dev)
        rb = q.run(args.steps, args.warmup, args.splits)
        bms = statistics.mean(rb["attn_ms"])
        result["bf16_twin"] = {
            "workload": "gqa8_16k_b32: 32 requests x 16384 tokens in the same 2 GiB as bf16 "
                        "(64 do not fit)",
            "tokens_per_s": 32 / (rb["ms_per_step"] * 1e-3),
            "ms_per_step": rb["ms_per_step"],
            "attn_GBps": q.bytes / (bms * 1e-3) / 1e9,
            "attn_frac": q.bytes / (bms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "num_splits": rb["splits"],
        }
        del q
        torch.cuda.empty_cache()
        # an extra that raises is recorded in the line, and the rest still run
        for name, fn in EXTRAS.items():
            try:
                result[name] = (concurrency_sweep(args, dev, head=p) if name == "concurrency_sweep"
                                else fn(args, dev))
            except Exception as e:   # noqa: BLE001 -- reported, not hidden
                log(f"extra {name} failed: {type(e).__name__}: {e}")
                result[name] = {"error": f"{type(e).__name__}: {e}"}
                torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
