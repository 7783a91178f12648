"""Multi-step decode with admission (paged_attention_fp8_amd/decode_loop.py):
every step's pool pages and attention against the oracle rebuilt from the
tokens the loop wrote; admission under a fixed pool budget (e4m3 runs twice
the requests of bf16); termination of a request whose page was handed on."""
import numpy as np
import pytest
import torch

import oracle
from paged_attention_fp8_amd import decode_loop as DL
from paged_attention_fp8_amd import ops
import types

from helpers import allclose_report, kv_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def _loop(kv_dtype, requests_pages, H=(8, 2), D=64, P=16, B=4, max_context=256, seed=0, record=True):
    Hq, Hkv = H
    elem = 1 if kv_dtype == ops.KV_FP8_E4M3 else 2
    pool_bytes = requests_pages * 2 * Hkv * P * D * elem
    ks = np.full(Hkv, 4.5 / 448, np.float32)
    vs = np.full(Hkv, 4.0 / 448, np.float32)
    return DL.DecodeLoop(kv_dtype, pool_bytes, Hq, Hkv, D, P, B, max_context, DEV, seed, ks, vs,
                         record=record)


def _check_against_oracle(loop: DL.DecodeLoop, kv_dtype):
    """Pool pages of the running requests are bit-exact and their attention
    output is within tolerance of the oracle, both rebuilt from the tokens
    the loop wrote."""
    running = [r for r in loop.slots if r is not None]
    if not running:
        return 0
    fp8 = kv_dtype == ops.KV_FP8_E4M3
    okv = oracle.KV_FP8 if fp8 else oracle.KV_BF16
    ks = loop.cache.k_scale.cpu().numpy() if fp8 else None
    vs = loop.cache.v_scale.cpu().numpy() if fp8 else None
    pool = oracle.Pool(okv, loop.num_pages, loop.Hkv, loop.P, loop.D, fill=0)
    table = np.full((len(running), loop.maxP), -1, np.int32)
    lens = np.zeros(len(running), np.int32)
    T = max(r.prompt_len + r.done for r in running)
    k = np.zeros((len(running), T, loop.Hkv, loop.D), np.uint16)
    v = np.zeros_like(k)
    for i, r in enumerate(running):
        kt, vt = loop.tokens_of(r.rid)
        L = kt.shape[0]
        table[i, :len(r.pages)] = r.pages
        lens[i] = L
        k[i, :L], v[i, :L] = kt, vt
    oracle.kv_write(pool, table, np.zeros(len(running), np.int32), lens, k, v, ks, vs)
    kp, vp = loop.cache.k_pool.cpu(), loop.cache.v_pool.cpu()
    if not fp8:
        kp, vp = kp.view(torch.int16).numpy().view(np.uint16), vp.view(torch.int16).numpy().view(np.uint16)
    else:
        kp, vp = kp.numpy(), vp.numpy()
    dev_pool = types.SimpleNamespace(k=kp, v=vp, kv_dtype=okv, P=loop.P, D=loop.D, Hkv=loop.Hkv)
    for i, r in enumerate(running):
        t = np.arange(lens[i])
        pages, slots_ = r.pages[t // loop.P], t % loop.P
        kd, vd = kv_rows(dev_pool, pages, slots_)
        kr, vr = kv_rows(pool, pages, slots_)
        assert np.array_equal(kd, kr), f"K of request {r.rid}"
        assert np.array_equal(vd, vr), f"V of request {r.rid}"
    slots = [r.slot for r in running]
    q = loop.last_q[slots].view(torch.int16).numpy().view(np.uint16)
    ro, rl = oracle.paged_attention(pool, q, table, lens, loop.sm, ks, vs)
    out = loop.out[slots].cpu().numpy()
    lse = loop.lse[slots].cpu().numpy()
    ok1, ma, mr = allclose_report(out, ro)
    ok2, la, _ = allclose_report(lse, rl)
    assert ok1 and ok2, (ma, mr, la)
    return len(running)


@pytest.mark.parametrize("kv_dtype", [ops.KV_FP8_E4M3, ops.KV_BF16], ids=["fp8", "bf16"])
def test_loop_matches_oracle_step_by_step(kv_dtype):
    say(f"decode loop vs oracle: dtype={kv_dtype}")
    loop = _loop(kv_dtype, requests_pages=24, seed=3)
    g = np.random.default_rng(5)
    for rid in range(9):
        loop.submit(DL.Request(rid, int(g.integers(1, 90)), int(g.integers(1, 7))))
    checked = 0
    for _ in range(60):
        st = loop.step()
        checked += _check_against_oracle(loop, kv_dtype)
        assert st.terminated == 0
        if not loop.queue and all(r is None for r in loop.slots):
            break
    assert len(loop.finished) == 9 and not any(r.terminated for r in loop.finished)
    assert len(loop.free) == loop.num_pages      # every page came back
    assert checked > 0


def test_same_budget_runs_twice_the_requests_in_e4m3():
    """A pool budget that holds 8 requests' pages in e4m3 holds 4 in bf16:
    with 8 requests waiting, e4m3 runs all 8 at once, bf16 runs 4 and queues 4."""
    say("decode loop: admission under one budget")
    res = {}
    for kv_dtype in (ops.KV_FP8_E4M3, ops.KV_BF16):
        elem = 1 if kv_dtype == ops.KV_FP8_E4M3 else 2
        per_req_pages = 8                                   # 128 tokens in 16-token pages
        budget = 8 * per_req_pages * 2 * 2 * 16 * 64 * 1    # 8 e4m3 requests
        loop = DL.DecodeLoop(kv_dtype, budget, 8, 2, 64, 16, 8, 128, DEV, 1,
                             np.full(2, 0.01, np.float32), np.full(2, 0.01, np.float32))
        assert loop.num_pages == 8 * per_req_pages // elem
        for rid in range(8):
            loop.submit(DL.Request(rid, 120, 8))
        st = loop.step()
        res[kv_dtype] = (st.active, st.waiting)
        while loop.queue or any(r is not None for r in loop.slots):
            loop.step()
        assert len(loop.finished) == 8
    assert res[ops.KV_FP8_E4M3] == (8, 0)
    assert res[ops.KV_BF16] == (4, 4)


def test_page_handed_on_terminates_its_request():
    """A page of a running request gets a new tag behind its back: the next
    step terminates exactly that request (nothing written, out 0, lse -inf);
    the others carry on and still match the oracle."""
    say("decode loop: termination on a stale page")
    loop = _loop(ops.KV_FP8_E4M3, requests_pages=40, seed=9)
    for rid in range(4):
        loop.submit(DL.Request(rid, 40 + 10 * rid, 6))
    loop.step()
    victim = loop.slots[2]
    assert victim is not None
    loop.reallocate_behind(victim, 1)
    st = loop.step()
    assert st.terminated == 1 and victim.terminated and victim.finished_at == st.step
    assert loop.status[victim.slot].item() == oracle.REQ_TAG_MISMATCH
    assert torch.all(loop.out[victim.slot] == 0) and torch.all(torch.isneginf(loop.lse[victim.slot]))
    assert _check_against_oracle(loop, ops.KV_FP8_E4M3) == 3
