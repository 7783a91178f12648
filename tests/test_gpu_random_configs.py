"""Seeded random configurations of the whole decode step (check, append,
attention) against the oracle: pool dtype, head dim, KV heads, query group,
page size, batch, ragged lengths (with exact page multiples and one-token
requests mixed in) and the split choice (library default, uniform splits or
the balanced partition) are drawn independently, at sizes the oracle finishes
in well under a second.  The bar is the attention tests': caches byte-equal
to the oracle's, outputs within 2e-3 + 1e-2 |oracle|."""
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


def _draw(n, seed=2026, batch=(1, 7)):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kv = int(g.choice([ops.KV_FP8_E4M3, ops.KV_BF16]))
        D = int(g.choice([64, 128]))
        Hkv = int(g.choice([1, 2, 3, 4, 8]))
        G = int(g.choice([1, 2, 3, 4, 5, 8, 16]))
        while Hkv * G > 64:
            G //= 2
        P = int(g.choice([16, 32, 64, 128, 256]))
        B = int(g.integers(*batch))
        lens = g.integers(1, 3000, B)
        lens[g.integers(0, B)] = P * int(g.integers(1, 12))      # an exact page multiple
        if B > 2:
            lens[g.integers(0, B)] = 1                           # a one-token request
        splits = g.choice(["default", "1", "2", "3", "5", "8", "-1", "-3", "-17", "balanced"])
        out.append((i, kv, D, Hkv, G, P, [int(x) for x in lens], str(splits)))
    return out


# 48 small batches, and 32 of 7-24 requests, whose grids (requests x KV
# heads x splits) are dealt to the XCDs in uneven ranges
CONFIGS = _draw(48) + [(48 + c[0],) + c[1:] for c in _draw(32, seed=2031, batch=(7, 25))]


def _id(c):
    i, kv, D, Hkv, G, P, lens, splits = c
    return f"{i}-{'fp8' if kv == ops.KV_FP8_E4M3 else 'bf16'}-d{D}-h{Hkv}x{G}-p{P}-b{len(lens)}-s{splits}"


@pytest.mark.parametrize("cfg", CONFIGS, ids=[_id(c) for c in CONFIGS])
def test_random_configuration_matches_oracle(cfg):
    i, kv, D, Hkv, G, P, lens, splits = cfg
    print(f"random config {_id(cfg)} lens={lens}", flush=True)
    w = I.Workload(f"random{i}", len(lens), Hkv * G, Hkv, D, P, 1, 3000, pool_factor=1.4)
    inp = I.make_decode_inputs(w, 500 + i, lengths=lens)
    step = H.build_step(inp, kv, DEV, poison=True)
    sm = 1.0 / math.sqrt(D)
    S = {"default": 0, "balanced": ops.BALANCED}.get(splits)
    S = int(splits) if S is None else S
    out, lse, status = H.decode_step(step, sm, S)
    torch.cuda.synchronize()
    assert np.all(status.cpu().numpy() == 0)
    ref = oracle_pool(inp, kv, poison=True)
    k, v = step.cache.k_pool.cpu(), step.cache.v_pool.cpu()
    if kv == ops.KV_BF16:
        k = k.view(torch.int16).numpy().view(np.uint16)
        v = v.view(torch.int16).numpy().view(np.uint16)
    else:
        k, v = k.numpy(), v.numpy()
    assert np.array_equal(k, ref.k) and np.array_equal(v, ref.v), "caches differ"
    ks = inp.k_scale if kv == ops.KV_FP8_E4M3 else None
    vs = inp.v_scale if kv == ops.KV_FP8_E4M3 else None
    ro, rl = oracle.paged_attention(ref, inp.q, inp.batch.page_table, inp.batch.context_lens, sm, ks, vs)
    ok1, ma, mr = allclose_report(out.cpu().numpy(), ro)
    ok2, la, _ = allclose_report(lse.cpu().numpy(), rl)
    print(f"  out max_abs={ma:.3e} max_rel={mr:.3e}; lse max_abs={la:.3e}", flush=True)
    assert ok1 and ok2


def _draw_fill(n, seed=2027):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kv = int(g.choice([ops.KV_FP8_E4M3, ops.KV_BF16]))
        D = int(g.choice([64, 128]))
        Hkv = int(g.choice([1, 2, 3, 8]))
        P = int(g.choice([16, 32, 64, 128, 256]))
        B = int(g.integers(1, 6))
        L = int(g.integers(P, 6 * P + 1))
        T = int(g.integers(1, 400))
        scale_exp = int(g.integers(-70, 70))      # per-head scales also far outside [2^-64, 2^64]
        out.append((i, kv, D, Hkv, P, B, L, T, scale_exp))
    return out


FILLS = _draw_fill(24)


@pytest.mark.parametrize("cfg", FILLS, ids=[f"{c[0]}-{'fp8' if c[1] == ops.KV_FP8_E4M3 else 'bf16'}"
                                            f"-d{c[2]}-h{c[3]}-p{c[4]}-b{c[5]}-T{c[7]}-s2^{c[8]}"
                                            for c in FILLS])
def test_random_fill_matches_oracle(cfg):
    """kv_quant_fill at random starts (negative and past the table included),
    counts (clipped at T), statuses and per-head scales: pools byte-equal."""
    i, kv, D, Hkv, P, B, L, T, scale_exp = cfg
    print(f"random fill {cfg}", flush=True)
    g = np.random.default_rng(900 + i)
    w = I.Workload(f"fill{i}", B, Hkv, Hkv, D, P, L, L, pool_factor=1.0)
    inp = I.make_decode_inputs(w, 700 + i)
    fp8 = kv == ops.KV_FP8_E4M3
    ks = (inp.k_scale * np.float32(2.0 ** scale_exp)).astype(np.float32)
    vs = (inp.v_scale * np.float32(2.0 ** -scale_exp)).astype(np.float32)
    cache = H.new_cache(w, inp.num_pages, kv, DEV, ks if fp8 else None, vs if fp8 else None)
    dbatch, _, _ = H.upload_batch(inp.batch, inp.pool, DEV)
    cap = inp.batch.max_pages * P
    start = g.integers(-P, cap + P, B).astype(np.int32)
    count = g.integers(0, T + 50, B).astype(np.int32)
    status = np.where(g.random(B) < 0.2, 2, 0).astype(np.int32)
    k_src = g.standard_normal((B, T, Hkv, D)).astype(np.float32) * np.float32(4.0)
    v_src = g.standard_normal((B, T, Hkv, D)).astype(np.float32) * np.float32(4.0)
    kb, vb = I.f32_to_bf16_bits(k_src), I.f32_to_bf16_bits(v_src)
    db = dbatch.with_status(torch.from_numpy(status).to(DEV))
    ops.kv_quant_fill(cache, db, torch.from_numpy(start).to(DEV), torch.from_numpy(count).to(DEV),
                      H.bf16_tensor(kb, DEV), H.bf16_tensor(vb, DEV))
    okv = oracle.KV_FP8 if fp8 else oracle.KV_BF16
    fill = H.FP8_NAN_CODE if fp8 else H.BF16_NAN_BITS
    ref = oracle.Pool(okv, inp.num_pages, Hkv, P, D, fill=fill)
    oracle.kv_write(ref, inp.batch.page_table, start, np.minimum(count, T), kb, vb,
                    ks if fp8 else None, vs if fp8 else None, status=status)
    k, v = cache.k_pool.cpu(), cache.v_pool.cpu()
    if fp8:
        k, v = k.numpy(), v.numpy()
    else:
        k = k.view(torch.int16).numpy().view(np.uint16)
        v = v.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(k, ref.k) and np.array_equal(v, ref.v)
